/*
 * ORACLE -- test infrastructure only.  Plain, slow, fp64 CPU reference of the
 * gated delta-rule recurrence.  Only tests/, __graft_entry__.smoke() and the
 * CPU-baseline leg of bench.py may build, load or call this file.  It shares
 * no code, header, table or helper with the GPU library.
 *
 * What it computes, token by token, for every (batch b, head h) on its own:
 *
 *   alpha_t = exp(log_alpha_t)            decay, scalar per head or one value
 *                                         per key channel (Gated DeltaNet-2,
 *                                         "Gated Delta Rule-2": D_t = Diag(alpha_t),
 *                                         channel-wise decay taken from KDA)
 *   if the preconditioner is on:
 *       A_t = A_{t-1} + k_t (.) k_t       running diagonal of the key Gram
 *                                         matrix, inclusive of k_t
 *       beta'_t = beta_t / (A_t + eps)    P_t = Diag(A_t)^-1 folded into the
 *                                         gain (Preconditioned DeltaNet,
 *                                         section 2.2 "diagonal preconditioner")
 *   else beta'_t = beta_t
 *   precond_mode 1 (stabilised, "Preconditioned DeltaNet" Eq. 9 as read
 *   here; the pages do not print the centring constant, the exponent base or
 *   the sign, so this form is a reading and its parity with the pages is
 *   unpinned):
 *       l_i = ln(A_t,i + eps), mu = mean_i l_i     log second moment, centred
 *       r_i = l_i - mu, s_i = r_i / (1 + |r_i|)    squashed into (-1, 1)
 *       B_i = x^(-s_i)                             in (1/x, x); larger A, smaller B
 *       beta'_t = beta_t (.) B_t
 *   gamma'_t = beta_t (raw) when gamma is "same as beta", else gamma_t
 *   kt = sqrt(beta'_t) (.) k_t            symmetric square-root gain on the
 *   vt = sqrt(gamma'_t) (.) v_t           key and the value (FG^2-GDN, 2.1;
 *                                         independent key/value gains, 2.2)
 *   Ad  = Diag(alpha_t) S_{t-1}           row i (key channel i) scaled
 *   u   = vt - Ad^T kt
 *   S_t = Ad + kt u^T                     = (I - kt kt^T) Diag(alpha_t) S_{t-1}
 *                                           + kt vt^T   (FG^2-GDN, 2.1)
 *   o_t = S_t^T q_t                       read-out with the updated state
 *
 * key_mode selects where the gains act (write key kw, read key kr, value vw;
 * every mode is S_t = Ad + kw (vw - Ad^T kr)^T = (I - kw kr^T) Ad + kw vw^T):
 *   0 symmetric   kw = kr = sqrt(beta') (.) k, vw = sqrt(gamma') (.) v   (above)
 *   1 erase gate  kw = k, kr = beta' (.) k, vw = gamma' (.) v
 *                 ("Gated DeltaNet-2" method 1: (I - k (b (.) k)^T) D S +
 *                 k (w (.) v)^T with erase gate b = beta', write gate w = gamma')
 *   2 write gate  kw = beta' (.) k, kr = k, vw = v if gamma is "same as beta"
 *                 (the gain rides on the write key), else gamma (.) v
 *                 ("Preconditioned DeltaNet" apply-to-key: the write key is
 *                 transformed, the read key is k)
 *
 * Layouts (row-major, contiguous): q, k [B,H,T,dk]; v, o [B,H,T,dv];
 * log_alpha [B,H,T] (scalar) or [B,H,T,dk] (vector); beta [B,H,T] or
 * [B,H,T,dk]; gamma [B,H,T] or [B,H,T,dv]; S0, ST [B,H,dk,dv]; A0, AT [B,H,dk].
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_ALPHA_NONE 0
#define OR_ALPHA_SCALAR 1
#define OR_ALPHA_VEC 2
#define OR_GATE_SCALAR 1
#define OR_GATE_VEC 2
#define OR_GAMMA_SAME 3
#define OR_KEY_SYMMETRIC 0
#define OR_KEY_ERASE_GATE 1
#define OR_KEY_WRITE_GATE 2
#define OR_PRECOND_INVERSE 0
#define OR_PRECOND_STABILISED 1

/* Returns 0 on success, -1 on a bad argument, -2 when out of memory. */
int oracle_delta_rule(int B, int H, int T, int dk, int dv,
                      const double *q, const double *k, const double *v,
                      int alpha_mode, const double *log_alpha,
                      int beta_mode, const double *beta,
                      int gamma_mode, const double *gamma,
                      double precond_eps, const double *A0, double *AT,
                      const double *S0, double *ST, double *o, int key_mode,
                      int precond_mode, double precond_x)
{
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    if (alpha_mode != OR_ALPHA_NONE && alpha_mode != OR_ALPHA_SCALAR &&
        alpha_mode != OR_ALPHA_VEC) return -1;
    if (beta_mode != OR_GATE_SCALAR && beta_mode != OR_GATE_VEC) return -1;
    if (gamma_mode != OR_GATE_SCALAR && gamma_mode != OR_GATE_VEC &&
        gamma_mode != OR_GAMMA_SAME) return -1;
    if (gamma_mode == OR_GAMMA_SAME && beta_mode == OR_GATE_VEC && dk != dv) return -1;
    if (alpha_mode != OR_ALPHA_NONE && !log_alpha) return -1;
    if (!beta || (gamma_mode != OR_GAMMA_SAME && !gamma)) return -1;
    if (key_mode != OR_KEY_SYMMETRIC && key_mode != OR_KEY_ERASE_GATE &&
        key_mode != OR_KEY_WRITE_GATE) return -1;
    if (precond_mode != OR_PRECOND_INVERSE && precond_mode != OR_PRECOND_STABILISED) return -1;
    if (precond_mode == OR_PRECOND_STABILISED && !(precond_x > 1.0)) return -1;

    const long BH = (long)B * H;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *A = (double *)malloc(sizeof(double) * (size_t)dk);
        double *al = (double *)malloc(sizeof(double) * (size_t)dk);
        double *kt = (double *)malloc(sizeof(double) * (size_t)dk);
        double *kr = (double *)malloc(sizeof(double) * (size_t)dk);
        double *vt = (double *)malloc(sizeof(double) * (size_t)dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *pb = (double *)malloc(sizeof(double) * (size_t)dk);
        if (!S || !A || !al || !kt || !kr || !vt || !u || !pb) {
#pragma omp atomic write
            failed = 1;
            free(S); free(A); free(al); free(kt); free(kr); free(vt); free(u); free(pb);
            continue;
        }
        if (S0) memcpy(S, S0 + bh * dk * dv, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);
        for (int i = 0; i < dk; ++i) A[i] = A0 ? A0[bh * dk + i] : 0.0;

        for (long t = 0; t < T; ++t) {
            const long tok = bh * T + t;
            const double *qt = q + tok * dk;
            const double *kk = k + tok * dk;
            const double *vv = v + tok * dv;

            /* decay */
            for (int i = 0; i < dk; ++i) {
                if (alpha_mode == OR_ALPHA_NONE) al[i] = 1.0;
                else if (alpha_mode == OR_ALPHA_SCALAR) al[i] = exp(log_alpha[tok]);
                else al[i] = exp(log_alpha[tok * dk + i]);
            }
            /* preconditioner coefficient per key channel */
            if (precond_eps >= 0.0) {
                for (int i = 0; i < dk; ++i) A[i] += kk[i] * kk[i];
                if (precond_mode == OR_PRECOND_STABILISED) {
                    double mu = 0.0;
                    for (int i = 0; i < dk; ++i) mu += log(A[i] + precond_eps);
                    mu /= dk;
                    for (int i = 0; i < dk; ++i) {
                        const double r = log(A[i] + precond_eps) - mu;
                        const double sq = r / (1.0 + fabs(r));
                        pb[i] = exp(-sq * log(precond_x));
                    }
                }
            }
            /* key-side gain, with the preconditioner folded in; kt is the
               write key and kr the read key */
            for (int i = 0; i < dk; ++i) {
                double b = (beta_mode == OR_GATE_SCALAR) ? beta[tok] : beta[tok * dk + i];
                if (precond_eps >= 0.0)
                    b = (precond_mode == OR_PRECOND_INVERSE) ? b / (A[i] + precond_eps) : b * pb[i];
                if (key_mode == OR_KEY_SYMMETRIC) {
                    kt[i] = sqrt(b) * kk[i];
                    kr[i] = kt[i];
                } else if (key_mode == OR_KEY_ERASE_GATE) {
                    kt[i] = kk[i];
                    kr[i] = b * kk[i];
                } else {
                    kt[i] = b * kk[i];
                    kr[i] = kk[i];
                }
            }
            /* value-side gain */
            for (int j = 0; j < dv; ++j) {
                double g;
                if (gamma_mode == OR_GAMMA_SAME)
                    g = (beta_mode == OR_GATE_SCALAR) ? beta[tok] : beta[tok * dk + j];
                else if (gamma_mode == OR_GATE_SCALAR) g = gamma[tok];
                else g = gamma[tok * dv + j];
                if (key_mode == OR_KEY_SYMMETRIC) vt[j] = sqrt(g) * vv[j];
                else if (key_mode == OR_KEY_WRITE_GATE && gamma_mode == OR_GAMMA_SAME) vt[j] = vv[j];
                else vt[j] = g * vv[j];
            }
            /* S <- Diag(alpha) S */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[(long)i * dv + j] *= al[i];
            /* u = vt - S^T kr */
            for (int j = 0; j < dv; ++j) u[j] = vt[j];
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) u[j] -= S[(long)i * dv + j] * kr[i];
            /* S <- S + kt u^T */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += kt[i] * u[j];
            /* o_t = S^T q_t */
            double *ot = o + tok * dv;
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) ot[j] += S[(long)i * dv + j] * qt[i];
        }
        if (ST) memcpy(ST + bh * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        if (AT) for (int i = 0; i < dk; ++i) AT[bh * dk + i] = A[i];
        free(S); free(A); free(al); free(kt); free(kr); free(vt); free(u); free(pb);
    }
    return failed ? -2 : 0;
}

/* Threads an OpenMP parallel region of the oracle uses (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
