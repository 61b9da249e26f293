/* Drives the argument validation of libpdn.so (the *_check and
 * *_workspace_size entry points; nothing is launched) under AddressSanitizer
 * and UndefinedBehaviorSanitizer, linked against a host-only build of the
 * library: valid arguments in every mode, each field pushed out of range, and
 * sizes at and beyond the limits where the size arithmetic could overflow.
 * Pointers are never dereferenced by these entry points. */
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
    printf("api sanitizer driver: %d argument sets, ABI version %d\n", calls, pdn_abi_version());
    return 0;
}
