/*
 * Test program (test infrastructure): drives libpdn.so through its C ABI alone
 * -- no Python, no torch -- and checks the results against the fp64 oracle
 * (oracle/recurrence.c, linked into this program only).
 *
 *   1. per-channel-gate prefill: bf16 q/k/v, dk = dv = 128, per-channel decay
 *      and key gain, per-token value gain, preconditioner with a start sum,
 *      erase-gate keys, a start state, caller-allocated workspace;
 *   2. scalar-gate prefill (Gated DeltaNet gating), bf16 output, no workspace;
 *   3. five decode steps against a resident fp32 state, write-gate keys;
 *   4. the backward of a prefill (fp32 q/k/v, dk = dv = 64, T = 70, per-channel
 *      decay and key gain, per-token value gain, write-gate keys, the
 *      preconditioner with a start sum, a start state and dST): every
 *      gradient against the oracle's backward;
 *   5. error paths: a workspace one byte short (prefill and backward), an
 *      unknown key mode, an unsupported value width in the backward.
 *
 * Inputs come from a counter-based generator (splitmix64 of a running index),
 * rounded to bf16 where the GPU reads bf16, and the same values (widened to
 * double) go to the oracle.  Exit status 0 when every check passes.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pdn.h"

int oracle_delta_rule(int B, int H, int T, int dk, int dv, const double *q, const double *k,
                      const double *v, int alpha_mode, const double *log_alpha, int beta_mode,
                      const double *beta, int gamma_mode, const double *gamma, double precond_eps,
                      const double *A0, double *AT, const double *S0, double *ST, double *o,
                      int key_mode, int precond_mode, double precond_x);

int oracle_delta_rule_bwd(int B, int H, int T, int dk, int dv, const double *q, const double *k,
                          const double *v, int alpha_mode, const double *log_alpha, int beta_mode,
                          const double *beta, int gamma_mode, const double *gamma,
                          double precond_eps, const double *A0, const double *S0, int key_mode,
                          int precond_mode, double precond_x, const double *dO, const double *dST,
                          double *dq, double *dk_out, double *dv_out, double *dlog_alpha, double *dbeta,
                          double *dgamma, double *dS0, double *dA0);

static int failures = 0;

#define HIP_CHECK(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)

/* splitmix64 of a counter -> uniform in [0, 1) */
static uint64_t counter = 0;
static double uniform01(void) {
    uint64_t z = (counter++) + 0x9E3779B97F4A7C15ull * 0x1234567ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static double normal01(void) { /* Box-Muller */
    double u1 = uniform01(), u2 = uniform01();
    if (u1 < 1e-300) u1 = 1e-300;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double neg_softplus(double x) { return -(x > 30.0 ? x : log1p(exp(x))); }

/* float -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t bf16_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* n values, rows of length d L2-normalised when norm != 0, rounded to bf16 */
static void fill_bf16(uint16_t *bits, double *val, long n, int d, int norm) {
    for (long r = 0; r < n / d; ++r) {
        double row[256], s = 0.0;
        for (int i = 0; i < d; ++i) { row[i] = normal01(); s += row[i] * row[i]; }
        for (int i = 0; i < d; ++i) {
            const double x = norm ? row[i] / sqrt(s) : row[i];
            bits[r * d + i] = bf16_bits((float)x);
            val[r * d + i] = bf16_value(bits[r * d + i]);
        }
    }
}
static void fill_f32(float *f, double *val, long n, double (*map)(double), double scale) {
    for (long i = 0; i < n; ++i) {
        f[i] = (float)(scale * map(normal01()));
        val[i] = f[i];
    }
}
static double ident(double x) { return x; }

static double rel_l2(const double *ref, const float *got, long n) {
    double num = 0.0, den = 0.0;
    for (long i = 0; i < n; ++i) {
        const double d = (double)got[i] - ref[i];
        num += d * d;
        den += ref[i] * ref[i];
    }
    return sqrt(num / (den > 0 ? den : 1.0));
}
static void check(const char *what, double err, double tol) {
    const int ok = err <= tol && err == err;
    printf("%-58s rel-L2 %.3e  (bound %.0e)  %s\n", what, err, tol, ok ? "ok" : "FAIL");
    if (!ok) ++failures;
}
static void expect_code(const char *what, int got, int want) {
    printf("%-58s %d (%s)  %s\n", what, got, pdn_strerror(got), got == want ? "ok" : "FAIL");
    if (got != want) ++failures;
}

static void *dmalloc(size_t n) {
    void *p = NULL;
    HIP_CHECK(hipMalloc(&p, n ? n : 16));
    return p;
}
static void *dcopy(const void *h, size_t n) {
    void *p = dmalloc(n);
    HIP_CHECK(hipMemcpy(p, h, n, hipMemcpyHostToDevice));
    return p;
}

/* ---- 1 and 2: prefill ---- */
static void prefill_case(int vec, hipStream_t st) {
    const int B = 1, H = 2, T = vec ? 100 : 150, dk = 128, dv = 128;
    const long nq = (long)B * H * T * dk, nv = (long)B * H * T * dv, nt = (long)B * H * T;
    const long ns = (long)B * H * dk * dv, na = (long)B * H * dk;
    uint16_t *qb = malloc(nq * 2), *kb = malloc(nq * 2), *vb = malloc(nv * 2);
    double *q = malloc(nq * 8), *k = malloc(nq * 8), *v = malloc(nv * 8);
    fill_bf16(qb, q, nq, dk, 1);
    fill_bf16(kb, k, nq, dk, 1);
    fill_bf16(vb, v, nv, dv, 0);
    const long nla = vec ? nq : nt, nbe = vec ? nq : nt;
    float *la_f = malloc(nla * 4), *be_f = malloc(nbe * 4), *ga_f = malloc(nt * 4);
    double *la = malloc(nla * 8), *be = malloc(nbe * 8), *ga = malloc(nt * 8);
    fill_f32(la_f, la, nla, neg_softplus, 1.0);
    fill_f32(be_f, be, nbe, sigmoid, 1.0);
    fill_f32(ga_f, ga, nt, sigmoid, 1.0);
    float *s0_f = malloc(ns * 4), *a0_f = malloc(na * 4);
    double *s0 = malloc(ns * 8), *a0 = malloc(na * 8);
    fill_f32(s0_f, s0, ns, ident, 0.1);
    for (long i = 0; i < na; ++i) { a0_f[i] = (float)(0.5 + uniform01()); a0[i] = a0_f[i]; }

    pdn_chunk_fwd_args a;
    memset(&a, 0, sizeof a);
    a.B = B; a.H = H; a.T = T; a.dk = dk; a.dv = dv;
    a.qkv_dtype = PDN_BF16;
    a.o_dtype = vec ? PDN_F32 : PDN_BF16;
    a.q = dcopy(qb, nq * 2); a.k = dcopy(kb, nq * 2); a.v = dcopy(vb, nv * 2);
    a.alpha_mode = vec ? PDN_ALPHA_VEC : PDN_ALPHA_SCALAR;
    a.log_alpha = dcopy(la_f, nla * 4);
    a.beta_mode = vec ? PDN_GATE_VEC : PDN_GATE_SCALAR;
    a.beta = dcopy(be_f, nbe * 4);
    a.gamma_mode = vec ? PDN_GATE_SCALAR : PDN_GAMMA_SAME_AS_BETA;
    a.gamma = vec ? dcopy(ga_f, nt * 4) : NULL;
    a.key_mode = vec ? PDN_KEY_ERASE_GATE : PDN_KEY_SYMMETRIC;
    a.precond_eps = vec ? 1e-6f : -1.0f;
    a.precond_A0 = vec ? dcopy(a0_f, na * 4) : NULL;
    a.precond_AT = vec ? dmalloc(na * 4) : NULL;
    a.S0 = dcopy(s0_f, ns * 4);
    a.ST = dmalloc(ns * 4);
    a.o = dmalloc(nv * (vec ? 4 : 2));
    size_t ws = 0;
    expect_code(vec ? "workspace size (per-channel gates)" : "workspace size (scalar gates)",
                pdn_chunk_fwd_workspace_size(&a, &ws), PDN_OK);
    if (vec ? ws == 0 : ws != 0) { printf("unexpected workspace size %zu  FAIL\n", ws); ++failures; }
    if (ws) {
        a.workspace = dmalloc(ws);
        a.workspace_bytes = ws - 1;
        expect_code("pdn_chunk_fwd with a workspace one byte short", pdn_chunk_fwd(&a, st), PDN_EWORKSPACE);
        a.workspace_bytes = ws;
    }
    expect_code(vec ? "pdn_chunk_fwd (per-channel gates, erase gate)" : "pdn_chunk_fwd (scalar gates)",
                pdn_chunk_fwd(&a, st), PDN_OK);
    HIP_CHECK(hipStreamSynchronize(st));

    double *o_ref = malloc(nv * 8), *s_ref = malloc(ns * 8), *a_ref = malloc(na * 8);
    if (oracle_delta_rule(B, H, T, dk, dv, q, k, v, a.alpha_mode, la, a.beta_mode, be, a.gamma_mode,
                          vec ? ga : NULL, vec ? 1e-6 : -1.0, vec ? a0 : NULL, vec ? a_ref : NULL, s0,
                          s_ref, o_ref, a.key_mode, PDN_PRECOND_INVERSE, 1.5) != 0) {
        printf("oracle failed  FAIL\n");
        ++failures;
        return;
    }
    float *o = malloc(nv * 4), *s = malloc(ns * 4), *at = malloc(na * 4);
    if (vec) {
        HIP_CHECK(hipMemcpy(o, a.o, nv * 4, hipMemcpyDeviceToHost));
        HIP_CHECK(hipMemcpy(at, a.precond_AT, na * 4, hipMemcpyDeviceToHost));
    } else {
        uint16_t *ob = malloc(nv * 2);
        HIP_CHECK(hipMemcpy(ob, a.o, nv * 2, hipMemcpyDeviceToHost));
        for (long i = 0; i < nv; ++i) o[i] = (float)bf16_value(ob[i]);
        free(ob);
    }
    HIP_CHECK(hipMemcpy(s, a.ST, ns * 4, hipMemcpyDeviceToHost));
    /* bf16 storage of o alone adds ~1.7e-3 of relative error */
    check(vec ? "  o vs oracle" : "  o (bf16) vs oracle", rel_l2(o_ref, o, nv), vec ? 2e-3 : 4e-3);
    check("  final state vs oracle", rel_l2(s_ref, s, ns), 2e-3);
    if (vec) check("  running k.k sum vs oracle", rel_l2(a_ref, at, na), 1e-6);

    hipFree((void *)a.q); hipFree((void *)a.k); hipFree((void *)a.v);
    hipFree((void *)a.log_alpha); hipFree((void *)a.beta);
    if (a.gamma) hipFree((void *)a.gamma);
    if (a.precond_A0) hipFree((void *)a.precond_A0);
    if (a.precond_AT) hipFree(a.precond_AT);
    hipFree((void *)a.S0); hipFree(a.ST); hipFree(a.o);
    if (a.workspace) hipFree(a.workspace);
    free(qb); free(kb); free(vb); free(q); free(k); free(v);
    free(la_f); free(be_f); free(ga_f); free(la); free(be); free(ga);
    free(s0_f); free(a0_f); free(s0); free(a0); free(o_ref); free(s_ref); free(a_ref);
    free(o); free(s); free(at);
}

/* ---- 3: decode ---- */
static void decode_case(hipStream_t st) {
    const int B = 3, H = 2, T = 5, dk = 128, dv = 128;
    const long nq = (long)B * H * T * dk, nv = (long)B * H * T * dv, ns = (long)B * H * dk * dv;
    const long nt = (long)B * H * T;
    uint16_t *qb = malloc(nq * 2), *kb = malloc(nq * 2), *vb = malloc(nv * 2);
    double *q = malloc(nq * 8), *k = malloc(nq * 8), *v = malloc(nv * 8);
    fill_bf16(qb, q, nq, dk, 1);
    fill_bf16(kb, k, nq, dk, 1);
    fill_bf16(vb, v, nv, dv, 0);
    float *la_f = malloc(nq * 4), *be_f = malloc(nq * 4), *ga_f = malloc(nt * 4), *s0_f = malloc(ns * 4);
    double *la = malloc(nq * 8), *be = malloc(nq * 8), *ga = malloc(nt * 8), *s0 = malloc(ns * 8);
    fill_f32(la_f, la, nq, neg_softplus, 1.0);
    fill_f32(be_f, be, nq, sigmoid, 1.0);
    fill_f32(ga_f, ga, nt, sigmoid, 1.0);
    fill_f32(s0_f, s0, ns, ident, 0.02);

    /* per-step slices: token t of every (b, h), contiguous [B, H, d] */
    const long bh = (long)B * H;
    uint16_t *qs = malloc(bh * dk * 2), *ks = malloc(bh * dk * 2), *vs = malloc(bh * dv * 2);
    float *las = malloc(bh * dk * 4), *bes = malloc(bh * dk * 4), *gas = malloc(bh * 4);
    void *dq = dmalloc(bh * dk * 2), *dk_ = dmalloc(bh * dk * 2), *dv_ = dmalloc(bh * dv * 2);
    void *dla = dmalloc(bh * dk * 4), *dbe = dmalloc(bh * dk * 4), *dga = dmalloc(bh * 4);
    void *dS = dcopy(s0_f, ns * 4), *dout = dmalloc(bh * dv * 4);
    float *o = malloc(nv * 4);
    for (int t = 0; t < T; ++t) {
        for (long i = 0; i < bh; ++i) {
            memcpy(qs + i * dk, qb + (i * T + t) * dk, dk * 2);
            memcpy(ks + i * dk, kb + (i * T + t) * dk, dk * 2);
            memcpy(vs + i * dv, vb + (i * T + t) * dv, dv * 2);
            memcpy(las + i * dk, la_f + (i * T + t) * dk, dk * 4);
            memcpy(bes + i * dk, be_f + (i * T + t) * dk, dk * 4);
            gas[i] = ga_f[i * T + t];
        }
        HIP_CHECK(hipMemcpy(dq, qs, bh * dk * 2, hipMemcpyHostToDevice));
        HIP_CHECK(hipMemcpy(dk_, ks, bh * dk * 2, hipMemcpyHostToDevice));
        HIP_CHECK(hipMemcpy(dv_, vs, bh * dv * 2, hipMemcpyHostToDevice));
        HIP_CHECK(hipMemcpy(dla, las, bh * dk * 4, hipMemcpyHostToDevice));
        HIP_CHECK(hipMemcpy(dbe, bes, bh * dk * 4, hipMemcpyHostToDevice));
        HIP_CHECK(hipMemcpy(dga, gas, bh * 4, hipMemcpyHostToDevice));
        pdn_decode_args d;
        memset(&d, 0, sizeof d);
        d.B = B; d.H = H; d.dk = dk; d.dv = dv;
        d.qkv_dtype = PDN_BF16; d.o_dtype = PDN_F32;
        d.q = dq; d.k = dk_; d.v = dv_;
        d.alpha_mode = PDN_ALPHA_VEC; d.log_alpha = dla;
        d.beta_mode = PDN_GATE_VEC; d.beta = dbe;
        d.gamma_mode = PDN_GATE_SCALAR; d.gamma = dga;
        d.key_mode = PDN_KEY_WRITE_GATE;
        d.precond_eps = -1.0f;
        d.S = dS; d.o = dout;
        const int rc = pdn_decode_step(&d, st);
        if (rc != PDN_OK) { expect_code("pdn_decode_step", rc, PDN_OK); return; }
        HIP_CHECK(hipStreamSynchronize(st));
        float *ot = malloc(bh * dv * 4);
        HIP_CHECK(hipMemcpy(ot, dout, bh * dv * 4, hipMemcpyDeviceToHost));
        for (long i = 0; i < bh; ++i) memcpy(o + (i * T + t) * dv, ot + i * dv, dv * 4);
        free(ot);
        if (t == 0) {
            d.key_mode = 7;
            expect_code("pdn_decode_step with an unknown key mode", pdn_decode_step(&d, st), PDN_EINVAL);
        }
    }
    double *o_ref = malloc(nv * 8), *s_ref = malloc(ns * 8);
    oracle_delta_rule(B, H, T, dk, dv, q, k, v, PDN_ALPHA_VEC, la, PDN_GATE_VEC, be, PDN_GATE_SCALAR, ga,
                      -1.0, NULL, NULL, s0, s_ref, o_ref, PDN_KEY_WRITE_GATE, PDN_PRECOND_INVERSE, 1.5);
    float *s = malloc(ns * 4);
    HIP_CHECK(hipMemcpy(s, dS, ns * 4, hipMemcpyDeviceToHost));
    printf("pdn_decode_step x %d (write gate)\n", T);
    check("  o vs oracle", rel_l2(o_ref, o, nv), 2e-3);
    check("  resident state vs oracle", rel_l2(s_ref, s, ns), 2e-3);
    hipFree(dq); hipFree(dk_); hipFree(dv_); hipFree(dla); hipFree(dbe); hipFree(dga);
    hipFree(dS); hipFree(dout);
    free(qb); free(kb); free(vb); free(q); free(k); free(v); free(la_f); free(be_f); free(ga_f);
    free(s0_f); free(la); free(be); free(ga); free(s0); free(qs); free(ks); free(vs); free(las);
    free(bes); free(gas); free(o); free(o_ref); free(s_ref); free(s);
}

/* ---- 4: backward ---- */
static void bwd_case(hipStream_t st) {
    const int B = 1, H = 2, T = 70, dk = 64, dv = 64;
    const long nq = (long)B * H * T * dk, nv = (long)B * H * T * dv, nt = (long)B * H * T;
    const long ns = (long)B * H * dk * dv, na = (long)B * H * dk;
    float *q_f = malloc(nq * 4), *k_f = malloc(nq * 4), *v_f = malloc(nv * 4);
    double *q = malloc(nq * 8), *k = malloc(nq * 8), *v = malloc(nv * 8);
    for (long r = 0; r < nq / dk; ++r) {
        double a[64], b[64], sa = 0.0, sb = 0.0;
        for (int i = 0; i < dk; ++i) { a[i] = normal01(); b[i] = normal01(); sa += a[i] * a[i]; sb += b[i] * b[i]; }
        for (int i = 0; i < dk; ++i) {
            q_f[r * dk + i] = (float)(a[i] / sqrt(sa)); q[r * dk + i] = q_f[r * dk + i];
            k_f[r * dk + i] = (float)(b[i] / sqrt(sb)); k[r * dk + i] = k_f[r * dk + i];
        }
    }
    fill_f32(v_f, v, nv, ident, 1.0);
    float *la_f = malloc(nq * 4), *be_f = malloc(nq * 4), *ga_f = malloc(nt * 4);
    double *la = malloc(nq * 8), *be = malloc(nq * 8), *ga = malloc(nt * 8);
    fill_f32(la_f, la, nq, neg_softplus, 1.0);
    fill_f32(be_f, be, nq, sigmoid, 1.0);
    fill_f32(ga_f, ga, nt, sigmoid, 1.0);
    float *s0_f = malloc(ns * 4), *a0_f = malloc(na * 4), *dO_f = malloc(nv * 4), *dST_f = malloc(ns * 4);
    double *s0 = malloc(ns * 8), *a0 = malloc(na * 8), *dO = malloc(nv * 8), *dST = malloc(ns * 8);
    fill_f32(s0_f, s0, ns, ident, 0.1);
    for (long i = 0; i < na; ++i) { a0_f[i] = (float)(0.5 + uniform01()); a0[i] = a0_f[i]; }
    fill_f32(dO_f, dO, nv, ident, 1.0);
    fill_f32(dST_f, dST, ns, ident, 1.0);

    pdn_chunk_bwd_args a;
    memset(&a, 0, sizeof a);
    a.fwd.B = B; a.fwd.H = H; a.fwd.T = T; a.fwd.dk = dk; a.fwd.dv = dv;
    a.fwd.qkv_dtype = PDN_F32;
    a.fwd.o_dtype = PDN_F32;
    a.fwd.q = dcopy(q_f, nq * 4); a.fwd.k = dcopy(k_f, nq * 4); a.fwd.v = dcopy(v_f, nv * 4);
    a.fwd.alpha_mode = PDN_ALPHA_VEC; a.fwd.log_alpha = dcopy(la_f, nq * 4);
    a.fwd.beta_mode = PDN_GATE_VEC; a.fwd.beta = dcopy(be_f, nq * 4);
    a.fwd.gamma_mode = PDN_GATE_SCALAR; a.fwd.gamma = dcopy(ga_f, nt * 4);
    a.fwd.key_mode = PDN_KEY_WRITE_GATE;
    a.fwd.precond_eps = 1e-6f;
    a.fwd.precond_mode = PDN_PRECOND_INVERSE;
    a.fwd.precond_A0 = dcopy(a0_f, na * 4);
    a.fwd.S0 = dcopy(s0_f, ns * 4);
    a.dO = dcopy(dO_f, nv * 4);
    a.dST = dcopy(dST_f, ns * 4);
    a.dq = dmalloc(nq * 4); a.dk = dmalloc(nq * 4); a.dv = dmalloc(nv * 4);
    a.dlog_alpha = dmalloc(nq * 4); a.dbeta = dmalloc(nq * 4); a.dgamma = dmalloc(nt * 4);
    a.dS0 = dmalloc(ns * 4); a.dA0 = dmalloc(na * 4);
    size_t ws = 0;
    expect_code("backward workspace size", pdn_chunk_bwd_workspace_size(&a, &ws), PDN_OK);
    a.workspace = dmalloc(ws);
    a.workspace_bytes = ws - 1;
    expect_code("pdn_chunk_bwd with a workspace one byte short", pdn_chunk_bwd(&a, st), PDN_EWORKSPACE);
    a.workspace_bytes = ws;
    a.fwd.dv = 48;
    expect_code("pdn_chunk_bwd with dv = 48", pdn_chunk_bwd(&a, st), PDN_EUNSUPPORTED);
    a.fwd.dv = dv;
    expect_code("pdn_chunk_bwd (vector gates, write gate, preconditioner)", pdn_chunk_bwd(&a, st), PDN_OK);
    HIP_CHECK(hipStreamSynchronize(st));

    double *r_dq = malloc(nq * 8), *r_dk = malloc(nq * 8), *r_dv = malloc(nv * 8);
    double *r_dla = malloc(nq * 8), *r_dbe = malloc(nq * 8), *r_dga = malloc(nt * 8);
    double *r_dS0 = malloc(ns * 8), *r_dA0 = malloc(na * 8);
    if (oracle_delta_rule_bwd(B, H, T, dk, dv, q, k, v, PDN_ALPHA_VEC, la, PDN_GATE_VEC, be,
                              PDN_GATE_SCALAR, ga, 1e-6, a0, s0, PDN_KEY_WRITE_GATE,
                              PDN_PRECOND_INVERSE, 1.5, dO, dST, r_dq, r_dk, r_dv, r_dla, r_dbe,
                              r_dga, r_dS0, r_dA0) != 0) {
        printf("oracle backward failed  FAIL\n");
        ++failures;
        return;
    }
    struct { const char *name; void *dev; const double *ref; long n; } g[] = {
        {"  dq vs oracle", a.dq, r_dq, nq}, {"  dk vs oracle", a.dk, r_dk, nq},
        {"  dv vs oracle", a.dv, r_dv, nv}, {"  d log alpha vs oracle", a.dlog_alpha, r_dla, nq},
        {"  dbeta vs oracle", a.dbeta, r_dbe, nq}, {"  dgamma vs oracle", a.dgamma, r_dga, nt},
        {"  dS0 vs oracle", a.dS0, r_dS0, ns}, {"  dA0 vs oracle", a.dA0, r_dA0, na}};
    float *h = malloc(nq * 4);
    for (int j = 0; j < 8; ++j) {
        HIP_CHECK(hipMemcpy(h, g[j].dev, g[j].n * 4, hipMemcpyDeviceToHost));
        /* fp32 arithmetic throughout; the start sum keeps the preconditioner well conditioned */
        check(g[j].name, rel_l2(g[j].ref, h, g[j].n), 1e-5);
        hipFree(g[j].dev);
    }
    free(h);
    hipFree((void *)a.fwd.q); hipFree((void *)a.fwd.k); hipFree((void *)a.fwd.v);
    hipFree((void *)a.fwd.log_alpha); hipFree((void *)a.fwd.beta); hipFree((void *)a.fwd.gamma);
    hipFree((void *)a.fwd.precond_A0); hipFree((void *)a.fwd.S0);
    hipFree((void *)a.dO); hipFree((void *)a.dST); hipFree(a.workspace);
    free(q_f); free(k_f); free(v_f); free(q); free(k); free(v); free(la_f); free(be_f); free(ga_f);
    free(la); free(be); free(ga); free(s0_f); free(a0_f); free(dO_f); free(dST_f); free(s0); free(a0);
    free(dO); free(dST); free(r_dq); free(r_dk); free(r_dv); free(r_dla); free(r_dbe); free(r_dga);
    free(r_dS0); free(r_dA0);
}

int main(void) {
    int ndev = 0;
    HIP_CHECK(hipGetDeviceCount(&ndev));
    if (ndev < 1) { fprintf(stderr, "no GPU\n"); return 2; }
    printf("libpdn ABI version %d\n", pdn_abi_version());
    if (pdn_abi_version() != PDN_ABI_VERSION) { printf("ABI version mismatch  FAIL\n"); ++failures; }
    hipStream_t st;
    HIP_CHECK(hipStreamCreate(&st));
    prefill_case(1, st);
    prefill_case(0, st);
    decode_case(st);
    bwd_case(st);
    HIP_CHECK(hipStreamDestroy(st));
    printf("%s\n", failures ? "FAILED" : "all C-ABI checks passed");
    return failures ? 1 : 0;
}
