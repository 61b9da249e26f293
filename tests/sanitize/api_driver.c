/* Drives the argument validation of libpdn.so (the *_check and
 * *_workspace_size entry points; nothing is launched) under AddressSanitizer
 * and UndefinedBehaviorSanitizer, linked against a host-only build of the
 * library: valid arguments in every mode, each field pushed out of range,
 * sizes at and beyond the limits where the size arithmetic could overflow, and
 * 200,000 valid argument sets with random fields mutated at random (each
 * answer one of the library's codes, the workspace sizes consistent with the
 * checks).  Pointers
 * are never dereferenced by these entry points. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pdn.h"

#define FAKE ((void *)(uintptr_t)0x10000)

static pdn_chunk_fwd_args chunk_ok(void) {
    pdn_chunk_fwd_args a;
    memset(&a, 0, sizeof(a));
    a.B = 2; a.H = 3; a.T = 100; a.dk = 128; a.dv = 128;
    a.qkv_dtype = PDN_BF16; a.o_dtype = PDN_F32;
    a.q = a.k = a.v = FAKE; a.o = FAKE;
    a.alpha_mode = PDN_ALPHA_VEC; a.log_alpha = (const float *)FAKE;
    a.beta_mode = PDN_GATE_VEC; a.beta = (const float *)FAKE;
    a.gamma_mode = PDN_GATE_VEC; a.gamma = (const float *)FAKE;
    a.precond_eps = -1.0f; a.precond_x = 1.5f;
    a.workspace = FAKE; a.workspace_bytes = (size_t)1 << 40;
    return a;
}

static int probe_chunk(pdn_chunk_fwd_args a) {
    size_t n = 0;
    int r1 = pdn_chunk_fwd_check(&a);
    int r2 = pdn_chunk_fwd_workspace_size(&a, &n);
    pdn_chunk_bwd_args b;
    memset(&b, 0, sizeof(b));
    b.fwd = a;
    b.dO = (const float *)FAKE; b.dq = b.dk = b.dv = (float *)FAKE;
    b.dlog_alpha = a.alpha_mode ? (float *)FAKE : NULL;
    b.dbeta = (float *)FAKE;
    b.dgamma = a.gamma_mode == PDN_GAMMA_SAME_AS_BETA ? NULL : (float *)FAKE;
    b.workspace = FAKE; b.workspace_bytes = (size_t)1 << 40;
    int r3 = pdn_chunk_bwd_check(&b);
    int r4 = pdn_chunk_bwd_workspace_size(&b, &n);
    return r1 + r2 + r3 + r4;  /* codes are only observed, not asserted here */
}

/* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", 2014): a counter-based generator, seeded, for the random
 * argument sets below */
static uint64_t rng_state = 0x5eed5eedULL;
static uint64_t rnd(void) {
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}
static int32_t rnd_int(void) {
    static const int32_t pick[] = {0, 1, 2, 3, -1, -2, 15, 16, 31, 32, 33, 48, 63, 64, 65, 96, 127, 128,
                                   129, 255, 256, 257, 512, 4096, 65536, 1 << 20, 1 << 30,
                                   0x7fffffff, (int32_t)0x80000000};
    const uint64_t r = rnd();
    return (r & 3) ? pick[(r >> 2) % (sizeof(pick) / sizeof(pick[0]))] : (int32_t)(r >> 32);
}
static int32_t rnd_enum(void) { return (int32_t)(rnd() % 7) - 1; }  /* -1 .. 5 */
static void *rnd_ptr(void) {
    static const uintptr_t pick[] = {0, 0x10000, 0x10008, 0x10010, 0x10004, 0x20000};
    return (void *)pick[rnd() % (sizeof(pick) / sizeof(pick[0]))];
}
static float rnd_float(void) {
    static const float pick[] = {-1.0f, 0.0f, 1e-6f, 1.0f, 1.5f, 2.0f, 2.5f, -0.0f, 1e30f, -1e30f,
                                 __builtin_nanf(""), __builtin_inff(), -__builtin_inff()};
    return pick[rnd() % (sizeof(pick) / sizeof(pick[0]))];
}
static int code_ok(int c) { return c == PDN_OK || (c <= -1 && c >= -5); }

/* random argument sets: a valid set in a random mode, then each field replaced
 * by a random value with probability 1/12 (so that both the accepting paths
 * and the rejections near them are reached).  The validation must answer
 * with one of its codes (no crash, no undefined behaviour under the
 * sanitizers), and a workspace size must come only for arguments that the
 * check accepts once given a valid workspace. */
#define MUT(field, value) do { if (rnd() % 12 == 0) (field) = (value); } while (0)
static int accepted = 0;  /* random sets the prefill check accepted */
static int fuzz(int n) {
    int bad = 0;
    for (int it = 0; it < n; ++it) {
        pdn_chunk_fwd_args a = chunk_ok();
        a.B = 1 + (int32_t)(rnd() % 4); a.H = 1 + (int32_t)(rnd() % 4); a.T = (int32_t)(rnd() % 300);
        a.dk = (rnd() & 1) ? 128 : 64; a.dv = 32 * (int32_t)(1 + rnd() % 8);
        a.qkv_dtype = (int32_t)(rnd() & 1); a.o_dtype = (int32_t)(rnd() & 1);
        a.alpha_mode = (int32_t)(rnd() % 3); a.log_alpha = a.alpha_mode ? (const float *)FAKE : NULL;
        a.beta_mode = 1 + (int32_t)(rnd() & 1);
        a.gamma_mode = 1 + (int32_t)(rnd() % 3);
        a.gamma = a.gamma_mode == PDN_GAMMA_SAME_AS_BETA ? NULL : (const float *)FAKE;
        if (a.gamma_mode == PDN_GAMMA_SAME_AS_BETA && a.beta_mode == PDN_GATE_VEC) a.dv = a.dk;
        a.precond_eps = (rnd() & 1) ? 1e-6f : -1.0f;
        if (rnd() & 1) { a.S0 = (const float *)FAKE; a.ST = (rnd() & 1) ? (float *)FAKE : NULL; }
        MUT(a.B, rnd_int()); MUT(a.H, rnd_int()); MUT(a.T, rnd_int());
        MUT(a.dk, rnd_int()); MUT(a.dv, rnd_int());
        MUT(a.qkv_dtype, rnd_enum()); MUT(a.o_dtype, rnd_enum());
        MUT(a.q, rnd_ptr()); MUT(a.k, rnd_ptr()); MUT(a.v, rnd_ptr());
        MUT(a.alpha_mode, rnd_enum()); MUT(a.log_alpha, (const float *)rnd_ptr());
        MUT(a.beta_mode, rnd_enum()); MUT(a.beta, (const float *)rnd_ptr());
        MUT(a.gamma_mode, rnd_enum()); MUT(a.gamma, (const float *)rnd_ptr());
        MUT(a.key_mode, rnd_enum());
        MUT(a.precond_eps, rnd_float()); MUT(a.precond_mode, rnd_enum()); MUT(a.precond_x, rnd_float());
        MUT(a.precond_A0, (const float *)rnd_ptr()); MUT(a.precond_AT, (float *)rnd_ptr());
        MUT(a.S0, (const float *)rnd_ptr()); MUT(a.ST, (float *)rnd_ptr());
        MUT(a.o, rnd_ptr()); MUT(a.workspace, rnd_ptr());
        MUT(a.workspace_bytes, (size_t)(rnd() >> (rnd() % 64)));
        size_t nbytes = 0;
        const int c1 = pdn_chunk_fwd_check(&a);
        const int c2 = pdn_chunk_fwd_workspace_size(&a, &nbytes);
        if (!code_ok(c1) || !code_ok(c2)) ++bad;
        if (c2 == PDN_OK) {
            /* the size query does not look at the workspace itself: with an
             * aligned one of exactly the size it returned the check passes,
             * and with one byte less it asks for more */
            pdn_chunk_fwd_args aw = a;
            aw.workspace = nbytes ? FAKE : NULL; aw.workspace_bytes = nbytes;
            if (pdn_chunk_fwd_check(&aw) != PDN_OK) ++bad;
            if (nbytes) {
                aw.workspace_bytes = nbytes - 1;
                if (pdn_chunk_fwd_check(&aw) != PDN_EWORKSPACE) ++bad;
            }
        }
        if (c1 == PDN_OK && c2 != PDN_OK) ++bad;
        accepted += c1 == PDN_OK;
        pdn_chunk_bwd_args b;
        memset(&b, 0, sizeof(b));
        b.fwd = a;
        b.dO = (const float *)FAKE; b.dq = b.dk = b.dv = (float *)FAKE;
        b.dlog_alpha = a.alpha_mode ? (float *)FAKE : NULL;
        b.dbeta = (float *)FAKE;
        b.dgamma = a.gamma_mode == PDN_GAMMA_SAME_AS_BETA ? NULL : (float *)FAKE;
        b.workspace = FAKE; b.workspace_bytes = (size_t)1 << 40;
        MUT(b.dO, (const float *)rnd_ptr()); MUT(b.dST, (const float *)rnd_ptr());
        MUT(b.dq, (float *)rnd_ptr()); MUT(b.dk, (float *)rnd_ptr()); MUT(b.dv, (float *)rnd_ptr());
        MUT(b.dlog_alpha, (float *)rnd_ptr()); MUT(b.dbeta, (float *)rnd_ptr());
        MUT(b.dgamma, (float *)rnd_ptr()); MUT(b.dS0, (float *)rnd_ptr()); MUT(b.dA0, (float *)rnd_ptr());
        MUT(b.workspace, rnd_ptr()); MUT(b.workspace_bytes, (size_t)(rnd() >> (rnd() % 64)));
        const int c3 = pdn_chunk_bwd_check(&b);
        const int c4 = pdn_chunk_bwd_workspace_size(&b, &nbytes);
        if (!code_ok(c3) || !code_ok(c4)) ++bad;
        if (c3 == PDN_OK && c4 != PDN_OK) ++bad;
        pdn_decode_args d;
        memset(&d, 0, sizeof(d));
        d.B = a.B; d.H = a.H; d.dk = a.dk; d.dv = a.dv;
        d.qkv_dtype = a.qkv_dtype; d.o_dtype = a.o_dtype;
        d.q = a.q; d.k = a.k; d.v = a.v;
        d.alpha_mode = a.alpha_mode; d.log_alpha = a.log_alpha;
        d.beta_mode = a.beta_mode; d.beta = a.beta;
        d.gamma_mode = a.gamma_mode; d.gamma = a.gamma;
        d.key_mode = a.key_mode; d.precond_eps = a.precond_eps;
        d.precond_mode = a.precond_mode; d.precond_x = a.precond_x;
        d.precond_A = a.precond_eps >= 0.0f ? (float *)FAKE : NULL; d.S = (float *)FAKE; d.o = FAKE;
        MUT(d.precond_A, (float *)rnd_ptr()); MUT(d.S, (float *)rnd_ptr()); MUT(d.o, rnd_ptr());
        if (!code_ok(pdn_decode_check(&d))) ++bad;
    }
    return bad;
}

int main(void) {
    int calls = 0;
    const int32_t sizes[] = {0, 1, 31, 32, 33, 4096, 65536, 1 << 20, 1 << 30, 0x7fffffff};
    const int32_t dims[] = {1, 16, 32, 48, 64, 128, 256, 512};
    for (int am = 0; am < 3; ++am)
        for (int bm = 1; bm <= 2; ++bm)
            for (int gm = 1; gm <= 3; ++gm)
                for (int pre = 0; pre < 2; ++pre)
                    for (int km = 0; km < 3; ++km)
                        for (int qd = 0; qd < 2; ++qd)
                            for (int di = 0; di < 8; ++di) {
                                pdn_chunk_fwd_args a = chunk_ok();
                                a.alpha_mode = am; a.beta_mode = bm; a.gamma_mode = gm;
                                if (gm == PDN_GAMMA_SAME_AS_BETA) a.gamma = NULL;
                                if (am == PDN_ALPHA_NONE) a.log_alpha = NULL;
                                a.precond_eps = pre ? 1e-6f : -1.0f;
                                a.precond_mode = pre > 0 && km == 1;
                                a.key_mode = km; a.qkv_dtype = qd;
                                a.dv = dims[di];
                                probe_chunk(a);
                                ++calls;
                            }
    for (int i = 0; i < 10; ++i)
        for (int j = 0; j < 10; ++j)
            for (int t = 0; t < 10; ++t) {
                pdn_chunk_fwd_args a = chunk_ok();
                a.B = sizes[i]; a.H = sizes[j]; a.T = sizes[t];
                probe_chunk(a);
                a.alpha_mode = PDN_ALPHA_SCALAR; a.beta_mode = PDN_GATE_SCALAR;
                a.gamma_mode = PDN_GAMMA_SAME_AS_BETA; a.gamma = NULL;
                probe_chunk(a);
                calls += 2;
            }
    for (int i = 0; i < 10; ++i)
        for (int j = 0; j < 10; ++j) {
            pdn_decode_args d;
            memset(&d, 0, sizeof(d));
            d.B = sizes[i]; d.H = sizes[j]; d.dk = 128; d.dv = 64;
            d.q = d.k = d.v = FAKE; d.o = FAKE; d.S = (float *)FAKE;
            d.alpha_mode = PDN_ALPHA_SCALAR; d.log_alpha = (const float *)FAKE;
            d.beta_mode = PDN_GATE_SCALAR; d.beta = (const float *)FAKE;
            d.gamma_mode = PDN_GAMMA_SAME_AS_BETA;
            d.precond_eps = -1.0f;
            pdn_decode_check(&d);
            ++calls;
        }
    pdn_chunk_fwd_check(NULL);
    pdn_decode_check(NULL);
    pdn_chunk_bwd_check(NULL);
    for (int c = -6; c <= 1; ++c) (void)pdn_strerror(c);
    const int nfuzz = 200000;
    const int bad = fuzz(nfuzz);
    calls += nfuzz;
    printf("api sanitizer driver: %d argument sets (%d random, %d of them accepted), %d inconsistent answers, "
           "ABI version %d\n", calls, nfuzz, accepted, bad, pdn_abi_version());
    return bad ? 1 : 0;
}
