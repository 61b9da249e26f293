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

/*
 * Backward pass (reverse mode) of the recurrence above, for the loss
 *
 *   L = sum_t <dO_t, o_t> + <dST, S_T>
 *
 * The gate-aware backward of "Gated DeltaNet-2" (method, the chunked
 * backward remark) asks for the gradients with respect to q, k, v, the
 * decay, the gains and the starting state; this is the plain definition of
 * those gradients: every forward step above, undone in reverse order.  Per
 * token t, with Ad = Diag(alpha_t) S_{t-1}, u = vw - Ad^T kr and
 * S_t = Ad + kw u^T, o_t = S_t^T q_t, given dS (the gradient with respect
 * to S_t, accumulated from later tokens):
 *
 *   dS   += q_t dO_t^T          dq_t = S_t dO_t
 *   dkw   = dS u                du   = dS^T kw
 *   dvw   = du                  dAd  = dS - kr du^T      dkr = -Ad du
 *   dalpha_i = sum_j dAd_ij S_{t-1,ij}                   dS_{t-1} = Diag(alpha_t) dAd
 *
 * then (dkw, dkr, dvw) go to (dk, dbeta', dgamma') by the key mode, beta' to
 * beta and the running second moment A_t by the preconditioner, and
 * d log_alpha = dalpha (.) alpha.  A_t = A_{t-1} + k_t (.) k_t is inclusive of
 * k_t, so dk_t also gets 2 k_t (.) sum_{s >= t} dA_s, and dA0 is that sum
 * over the whole sequence.  States are recomputed from checkpoints every
 * OR_CKPT tokens.
 *
 * Outputs (all written, zero where a gate has no gradient): dq, dk
 * [B,H,T,dk]; dv [B,H,T,dv]; dlog_alpha in the shape of log_alpha (unused
 * when alpha_mode is NONE); dbeta in the shape of beta; dgamma in the shape
 * of gamma (unused when gamma is "same as beta": that gradient is added to
 * dbeta); dS0 [B,H,dk,dv]; dA0 [B,H,dk] (preconditioner only, may be NULL).
 * dST may be NULL (zero).  In the symmetric key mode the gradient of
 * sqrt(beta') is unbounded at beta' = 0 (and likewise for gamma').
 */
#define OR_CKPT 64

int oracle_delta_rule_bwd(int B, int H, int T, int dk, int dv,
                          const double *q, const double *k, const double *v,
                          int alpha_mode, const double *log_alpha,
                          int beta_mode, const double *beta,
                          int gamma_mode, const double *gamma,
                          double precond_eps, const double *A0, const double *S0,
                          int key_mode, int precond_mode, double precond_x,
                          const double *dO, const double *dST,
                          double *dq, double *dk_out, double *dv_out,
                          double *dlog_alpha, double *dbeta, double *dgamma,
                          double *dS0, double *dA0)
{
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    if (alpha_mode != OR_ALPHA_NONE && alpha_mode != OR_ALPHA_SCALAR &&
        alpha_mode != OR_ALPHA_VEC) return -1;
    if (beta_mode != OR_GATE_SCALAR && beta_mode != OR_GATE_VEC) return -1;
    if (gamma_mode != OR_GATE_SCALAR && gamma_mode != OR_GATE_VEC &&
        gamma_mode != OR_GAMMA_SAME) return -1;
    if (gamma_mode == OR_GAMMA_SAME && beta_mode == OR_GATE_VEC && dk != dv) return -1;
    if (alpha_mode != OR_ALPHA_NONE && (!log_alpha || !dlog_alpha)) return -1;
    if (!beta || !dbeta || (gamma_mode != OR_GAMMA_SAME && (!gamma || !dgamma))) return -1;
    if (key_mode != OR_KEY_SYMMETRIC && key_mode != OR_KEY_ERASE_GATE &&
        key_mode != OR_KEY_WRITE_GATE) return -1;
    if (precond_mode != OR_PRECOND_INVERSE && precond_mode != OR_PRECOND_STABILISED) return -1;
    if (precond_mode == OR_PRECOND_STABILISED && !(precond_x > 1.0)) return -1;
    if (!dO || !dq || !dk_out || !dv_out || !dS0) return -1;

    const long BH = (long)B * H;
    const long SZ = (long)dk * dv;
    const int nck = (T + OR_CKPT - 1) / OR_CKPT;
    const int pre = precond_eps >= 0.0;
    const double lnx = precond_mode == OR_PRECOND_STABILISED ? log(precond_x) : 0.0;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        /* per-token gates: alpha, raw erase gain, gain with the preconditioner
           folded in, value gain, and A_t */
        const long Tl = T > 0 ? T : 1;
        double *al = (double *)malloc(sizeof(double) * (size_t)(Tl * dk));
        double *braw = (double *)malloc(sizeof(double) * (size_t)(Tl * dk));
        double *bp = (double *)malloc(sizeof(double) * (size_t)(Tl * dk));
        double *Acc = (double *)malloc(sizeof(double) * (size_t)(Tl * dk));
        double *gv = (double *)malloc(sizeof(double) * (size_t)(Tl * dv));
        double *ck = (double *)malloc(sizeof(double) * (size_t)((nck + 1) * SZ));
        double *blk = (double *)malloc(sizeof(double) * (size_t)((OR_CKPT + 1) * SZ));
        double *dS = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *Ad = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *vec = (double *)malloc(sizeof(double) * (size_t)(6 * dk + 4 * dv));
        if (!al || !braw || !bp || !Acc || !gv || !ck || !blk || !dS || !Ad || !vec) {
#pragma omp atomic write
            failed = 1;
            free(al); free(braw); free(bp); free(Acc); free(gv); free(ck); free(blk);
            free(dS); free(Ad); free(vec);
            continue;
        }
        double *kw = vec, *kr = vec + dk, *dkw = vec + 2 * dk, *dkr = vec + 3 * dk;
        double *dAcc = vec + 4 * dk, *dbp = vec + 5 * dk;
        double *vw = vec + 6 * dk, *u = vw + dv, *du = u + dv, *dgv = du + dv;

        /* gates of every token (the forward's steps, in its order) */
        for (long t = 0; t < T; ++t) {
            const long tok = bh * T + t;
            const double *kk = k + tok * dk;
            for (int i = 0; i < dk; ++i) {
                if (alpha_mode == OR_ALPHA_NONE) al[t * dk + i] = 1.0;
                else if (alpha_mode == OR_ALPHA_SCALAR) al[t * dk + i] = exp(log_alpha[tok]);
                else al[t * dk + i] = exp(log_alpha[tok * dk + i]);
                const double prev = t > 0 ? Acc[(t - 1) * dk + i] : (A0 ? A0[bh * dk + i] : 0.0);
                Acc[t * dk + i] = prev + kk[i] * kk[i];
                braw[t * dk + i] = (beta_mode == OR_GATE_SCALAR) ? beta[tok] : beta[tok * dk + i];
            }
            double mu = 0.0;
            if (pre && precond_mode == OR_PRECOND_STABILISED) {
                for (int i = 0; i < dk; ++i) mu += log(Acc[t * dk + i] + precond_eps);
                mu /= dk;
            }
            for (int i = 0; i < dk; ++i) {
                double b = braw[t * dk + i];
                if (pre) {
                    const double a = Acc[t * dk + i] + precond_eps;
                    if (precond_mode == OR_PRECOND_INVERSE) b /= a;
                    else {
                        const double r = log(a) - mu;
                        b *= exp(-(r / (1.0 + fabs(r))) * lnx);
                    }
                }
                bp[t * dk + i] = b;
            }
            for (int j = 0; j < dv; ++j) {
                if (gamma_mode == OR_GAMMA_SAME)
                    gv[t * dv + j] = (beta_mode == OR_GATE_SCALAR) ? beta[tok] : beta[tok * dk + j];
                else if (gamma_mode == OR_GATE_SCALAR) gv[t * dv + j] = gamma[tok];
                else gv[t * dv + j] = gamma[tok * dv + j];
            }
        }

/* write key, read key and written value of token t */
#define OR_KEYS(t)                                                                   \
    do {                                                                             \
        const double *kk_ = k + (bh * T + (t)) * dk;                                 \
        const double *vv_ = v + (bh * T + (t)) * dv;                                 \
        for (int i = 0; i < dk; ++i) {                                               \
            const double b_ = bp[(t) * dk + i];                                      \
            if (key_mode == OR_KEY_SYMMETRIC) { kw[i] = sqrt(b_) * kk_[i]; kr[i] = kw[i]; } \
            else if (key_mode == OR_KEY_ERASE_GATE) { kw[i] = kk_[i]; kr[i] = b_ * kk_[i]; } \
            else { kw[i] = b_ * kk_[i]; kr[i] = kk_[i]; }                            \
        }                                                                            \
        for (int j = 0; j < dv; ++j) {                                               \
            const double g_ = gv[(t) * dv + j];                                      \
            if (key_mode == OR_KEY_SYMMETRIC) vw[j] = sqrt(g_) * vv_[j];             \
            else if (key_mode == OR_KEY_WRITE_GATE && gamma_mode == OR_GAMMA_SAME) vw[j] = vv_[j]; \
            else vw[j] = g_ * vv_[j];                                                \
        }                                                                            \
    } while (0)

/* S_out = one forward step of S_in with token t (Ad and u left set) */
#define OR_STEP(S_in, S_out, t)                                                      \
    do {                                                                             \
        OR_KEYS(t);                                                                  \
        for (int i = 0; i < dk; ++i)                                                 \
            for (int j = 0; j < dv; ++j) Ad[(long)i * dv + j] = al[(t) * dk + i] * (S_in)[(long)i * dv + j]; \
        for (int j = 0; j < dv; ++j) u[j] = vw[j];                                   \
        for (int i = 0; i < dk; ++i)                                                 \
            for (int j = 0; j < dv; ++j) u[j] -= Ad[(long)i * dv + j] * kr[i];      \
        for (int i = 0; i < dk; ++i)                                                 \
            for (int j = 0; j < dv; ++j) (S_out)[(long)i * dv + j] = Ad[(long)i * dv + j] + kw[i] * u[j]; \
    } while (0)

        /* forward: checkpoint c holds the state before token c * OR_CKPT */
        if (S0) memcpy(ck, S0 + bh * SZ, sizeof(double) * (size_t)SZ);
        else memset(ck, 0, sizeof(double) * (size_t)SZ);
        for (int c = 0; c < nck; ++c) {
            memcpy(blk, ck + (long)c * SZ, sizeof(double) * (size_t)SZ);
            const long t0 = (long)c * OR_CKPT, t1 = t0 + OR_CKPT < T ? t0 + OR_CKPT : T;
            for (long t = t0; t < t1; ++t) {
                OR_STEP(blk, blk, t);
            }
            memcpy(ck + (long)(c + 1) * SZ, blk, sizeof(double) * (size_t)SZ);
        }

        /* backward */
        if (dST) memcpy(dS, dST + bh * SZ, sizeof(double) * (size_t)SZ);
        else memset(dS, 0, sizeof(double) * (size_t)SZ);
        for (int i = 0; i < dk; ++i) dAcc[i] = 0.0;
        for (int c = nck - 1; c >= 0; --c) {
            const long t0 = (long)c * OR_CKPT, t1 = t0 + OR_CKPT < T ? t0 + OR_CKPT : T;
            /* blk[m] = state before token t0 + m */
            memcpy(blk, ck + (long)c * SZ, sizeof(double) * (size_t)SZ);
            for (long t = t0; t < t1; ++t) {
                OR_STEP(blk + (t - t0) * SZ, blk + (t - t0 + 1) * SZ, t);
            }
            for (long t = t1 - 1; t >= t0; --t) {
                const long tok = bh * T + t;
                const double *Sp = blk + (t - t0) * SZ;     /* S_{t-1} */
                const double *St = blk + (t - t0 + 1) * SZ; /* S_t */
                OR_STEP(Sp, blk + (t - t0 + 1) * SZ, t);    /* sets Ad, u, keys (S_t unchanged) */
                const double *dOt = dO + tok * dv;
                const double *qt = q + tok * dk;
                const double *kk = k + tok * dk;
                const double *vv = v + tok * dv;
                /* o_t = S_t^T q_t */
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        dS[(long)i * dv + j] += qt[i] * dOt[j];
                        acc += St[(long)i * dv + j] * dOt[j];
                    }
                    dq[tok * dk + i] = acc;
                }
                /* S_t = Ad + kw u^T */
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += dS[(long)i * dv + j] * u[j];
                    dkw[i] = acc;
                }
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < dk; ++i) acc += dS[(long)i * dv + j] * kw[i];
                    du[j] = acc;
                }
                /* u = vw - Ad^T kr: dAd = dS - kr du^T, dkr = -Ad du */
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += Ad[(long)i * dv + j] * du[j];
                    dkr[i] = -acc;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) dS[(long)i * dv + j] -= kr[i] * du[j];
                /* Ad = Diag(alpha) S_{t-1} */
                double dla_sum = 0.0;
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += dS[(long)i * dv + j] * Sp[(long)i * dv + j];
                    const double a = al[t * dk + i];
                    if (alpha_mode == OR_ALPHA_VEC) dlog_alpha[tok * dk + i] = acc * a;
                    dla_sum += acc * a;
                    for (int j = 0; j < dv; ++j) dS[(long)i * dv + j] *= a;
                }
                if (alpha_mode == OR_ALPHA_SCALAR) dlog_alpha[tok] = dla_sum;
                /* keys and value to k, v, beta', gamma' */
                for (int i = 0; i < dk; ++i) {
                    const double b = bp[t * dk + i];
                    double dki, dbi;
                    if (key_mode == OR_KEY_SYMMETRIC) {
                        const double sb = sqrt(b);
                        dki = (dkw[i] + dkr[i]) * sb;
                        dbi = (dkw[i] + dkr[i]) * kk[i] * 0.5 / sb;
                    } else if (key_mode == OR_KEY_ERASE_GATE) {
                        dki = dkw[i] + dkr[i] * b;
                        dbi = dkr[i] * kk[i];
                    } else {
                        dki = dkw[i] * b + dkr[i];
                        dbi = dkw[i] * kk[i];
                    }
                    dk_out[tok * dk + i] = dki;
                    dbp[i] = dbi;
                }
                for (int j = 0; j < dv; ++j) {
                    const double g = gv[t * dv + j];
                    if (key_mode == OR_KEY_SYMMETRIC) {
                        const double sg = sqrt(g);
                        dv_out[tok * dv + j] = du[j] * sg;
                        dgv[j] = du[j] * vv[j] * 0.5 / sg;
                    } else if (key_mode == OR_KEY_WRITE_GATE && gamma_mode == OR_GAMMA_SAME) {
                        dv_out[tok * dv + j] = du[j];
                        dgv[j] = 0.0;
                    } else {
                        dv_out[tok * dv + j] = du[j] * g;
                        dgv[j] = du[j] * vv[j];
                    }
                }
                /* beta' to the raw gain and A_t */
                if (pre) {
                    if (precond_mode == OR_PRECOND_INVERSE) {
                        for (int i = 0; i < dk; ++i) {
                            const double a = Acc[t * dk + i] + precond_eps;
                            dAcc[i] += -dbp[i] * braw[t * dk + i] / (a * a);
                            dbp[i] /= a;
                        }
                    } else {
                        /* B_i = x^-s_i, s = r / (1 + |r|), r_i = ln(A_i + eps) - mean */
                        double mu = 0.0;
                        for (int i = 0; i < dk; ++i) mu += log(Acc[t * dk + i] + precond_eps);
                        mu /= dk;
                        double mean_dr = 0.0;
                        for (int i = 0; i < dk; ++i) {
                            const double r = log(Acc[t * dk + i] + precond_eps) - mu;
                            const double Bi = exp(-(r / (1.0 + fabs(r))) * lnx);
                            const double dBi = dbp[i] * braw[t * dk + i];
                            const double dsi = -dBi * Bi * lnx;
                            const double den = 1.0 + fabs(r);
                            kw[i] = dsi / (den * den); /* dr_i (kw is free now) */
                            mean_dr += kw[i];
                            dbp[i] *= Bi;
                        }
                        mean_dr /= dk;
                        for (int i = 0; i < dk; ++i)
                            dAcc[i] += (kw[i] - mean_dr) / (Acc[t * dk + i] + precond_eps);
                    }
                    for (int i = 0; i < dk; ++i) dk_out[tok * dk + i] += 2.0 * kk[i] * dAcc[i];
                }
                /* raw gains */
                if (beta_mode == OR_GATE_SCALAR) {
                    double acc = 0.0;
                    for (int i = 0; i < dk; ++i) acc += dbp[i];
                    if (gamma_mode == OR_GAMMA_SAME)
                        for (int j = 0; j < dv; ++j) acc += dgv[j];
                    dbeta[tok] = acc;
                } else {
                    for (int i = 0; i < dk; ++i)
                        dbeta[tok * dk + i] = dbp[i] + (gamma_mode == OR_GAMMA_SAME ? dgv[i] : 0.0);
                }
                if (gamma_mode == OR_GATE_SCALAR) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += dgv[j];
                    dgamma[tok] = acc;
                } else if (gamma_mode == OR_GATE_VEC) {
                    for (int j = 0; j < dv; ++j) dgamma[tok * dv + j] = dgv[j];
                }
            }
        }
        memcpy(dS0 + bh * SZ, dS, sizeof(double) * (size_t)SZ);
        if (dA0 && pre)
            for (int i = 0; i < dk; ++i) dA0[bh * dk + i] = dAcc[i];
#undef OR_STEP
#undef OR_KEYS
        free(al); free(braw); free(bp); free(Acc); free(gv); free(ck); free(blk);
        free(dS); free(Ad); free(vec);
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
