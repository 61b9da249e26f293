/*
 * pdn.h -- C ABI of the MI355X (gfx950) gated delta-rule library (libpdn.so).
 *
 * The operation (per batch b and head h, key width dk, value width dv):
 *
 *   state S in R^{dk x dv};  for t = 1..T:
 *     alpha_t = exp(log_alpha_t)                 decay, scalar or per key channel
 *     beta'_t = beta_t (.) P(A_t),               when the diagonal preconditioner
 *       A_t = A_{t-1} + k_t (.) k_t              is on (A_t includes k_t); else beta_t
 *       P = 1 / (A_t + eps)                      (PDN_PRECOND_INVERSE), or
 *       P = x^-(r / (1 + |r|)),                  (PDN_PRECOND_STABILISED)
 *         r = ln(A_t + eps) - mean over the dk channels of ln(A_t + eps)
 *     kt = sqrt(beta'_t) (.) k_t,  vt = sqrt(gamma_t) (.) v_t
 *     S_t = Diag(alpha_t) S_{t-1} + kt (vt - (Diag(alpha_t) S_{t-1})^T kt)^T
 *     o_t = S_t^T q_t
 *
 * Sources (titles of the pages this follows):
 *   - "FG^2-GDN: Enhancing Long-Context Gated Delta Networks with Doubly
 *     Fine-Grained Control", technical summary 2.1 (symmetric sqrt(beta) on key
 *     and value, S_t = (I - kt kt^T) Diag(alpha_t) S_{t-1} + kt vt^T) and 2.2
 *     (independent key-side and value-side gains).
 *   - "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention",
 *     method section 1 (channel-wise decay D_t = Diag(alpha_t) before the erase;
 *     reduction to KDA / Gated DeltaNet for tied scalar gates) and section 3
 *     (chunkwise WY form with a lower-triangular (I+T)^-1 solve).
 *   - "Preconditioned DeltaNet: Curvature-aware Sequence Modeling for Linear
 *     Recurrences", section 2.2 / 2B (running diagonal A_t = A_{t-1} + k_t (.) k_t,
 *     P_t = Diag(A_t)^-1), folded here into the erase gain beta; Eq. 9 for the
 *     stabilised coefficient (log space, centring, the squash r / (1 + |r|),
 *     values in [1/x, x]).  The pages do not print the centring constant, the
 *     base or the sign; the mean of ln(A + eps) over the channels and x^-s are
 *     this library's reading.
 *   gamma is never preconditioned; "gamma same as beta" means the raw beta.
 *   There is no 1/sqrt(dk) scaling inside the op.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (HBM), row-major and contiguous,
 *     owned by the caller.  The library allocates nothing and keeps no mutable
 *     global state; it never frees or retains caller memory.
 *   - Work is queued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Outputs are valid once the stream is synchronised.
 *     The stream must belong to the current HIP device, the one whose memory
 *     the pointers address: grids are sized for the current device, and
 *     pdn_chunk_fwd_noalloc takes its scratch there.
 *   - The calls only launch kernels (no allocation, memset or copy), so they
 *     can be captured into a HIP graph and replayed.
 *   - Arguments are validated on the host BEFORE any launch; an invalid call
 *     returns a negative PDN_E* code, touches no memory and launches nothing.
 *     No C++ exception crosses this boundary.
 *   - Calls that share an output (o, ST, S, precond_A) must not overlap.
 */
#ifndef PDN_H
#define PDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PDN_ABI_VERSION 5

/* Return codes. */
#define PDN_OK 0
#define PDN_EINVAL (-1)        /* null pointer, bad size, bad enum value          */
#define PDN_EUNSUPPORTED (-2)  /* valid request outside what the kernels handle   */
#define PDN_EWORKSPACE (-3)    /* workspace missing or smaller than required      */
#define PDN_EHIP (-4)          /* the HIP runtime reported an error on launch     */
#define PDN_ESCRATCH (-5)      /* pdn_chunk_fwd_noalloc: the call needs more than
                                  PDN_NOALLOC_SCRATCH_BYTES of scratch          */

/* Element types of q, k, v and o. */
#define PDN_F32 0
#define PDN_BF16 1

/* Decay: none (alpha == 1), one scalar per (b,h,t), or one per key channel. */
#define PDN_ALPHA_NONE 0
#define PDN_ALPHA_SCALAR 1
#define PDN_ALPHA_VEC 2

/* Gains: one scalar per (b,h,t), one per channel, or (gamma only) raw beta. */
#define PDN_GATE_SCALAR 1
#define PDN_GATE_VEC 2
#define PDN_GAMMA_SAME_AS_BETA 3

/* Read / write key modes.  Every mode is S_t = A + kw (vw - A^T kr)^T with
 * A = Diag(alpha_t) S_{t-1} and beta' the erase gain with the preconditioner
 * folded in:
 *   SYMMETRIC   kw = kr = sqrt(beta') (.) k, vw = sqrt(gamma') (.) v
 *               ("FG^2-GDN" 2.1; the default, value 0)
 *   ERASE_GATE  kw = k, kr = beta' (.) k, vw = gamma' (.) v
 *               ("Gated DeltaNet-2" method 1: (I - k (b (.) k)^T) D S + k (w (.) v)^T)
 *   WRITE_GATE  kw = beta' (.) k, kr = k, vw = v when gamma is "same as beta"
 *               (the gain rides on the write key), else gamma (.) v
 *               ("Preconditioned DeltaNet" 2.2: apply-to-key write key)
 * The asymmetric modes need bf16 q/k/v with dk == 128 and dv % 32 == 0 in
 * the prefill (PDN_EUNSUPPORTED otherwise); decode takes every mode. */
#define PDN_KEY_SYMMETRIC 0
#define PDN_KEY_ERASE_GATE 1
#define PDN_KEY_WRITE_GATE 2

/* Preconditioner coefficient (when precond_eps >= 0). */
#define PDN_PRECOND_INVERSE 0     /* 1 / (A_t + eps) */
#define PDN_PRECOND_STABILISED 1  /* x^-(r/(1+|r|)), see above; needs 1 < precond_x <= 2,
                                     and in the prefill bf16 q/k/v with dk == 128 and
                                     dv % 32 == 0 (PDN_EUNSUPPORTED otherwise) */

/*
 * Prefill over whole sequences, chunkwise-parallel on the GPU.
 *
 *   B, H, T, dk, dv   sizes.  B, H >= 1; T >= 0 (T == 0 copies S0 to ST and
 *                     A0 to AT; the q/k/v/o/gate pointers may then be NULL);
 *                     dk in {64, 128}; dv a multiple of 16 and <= 256, and a
 *                     multiple of 32 when any gate is per-channel or the
 *                     preconditioner is on.  Every pointer must be 16-byte
 *                     aligned (PDN_EINVAL otherwise).
 *   qkv_dtype         PDN_F32 or PDN_BF16: element type of q, k, v.
 *   o_dtype           PDN_F32 (default) or PDN_BF16.
 *   q, k              [B,H,T,dk].      v: [B,H,T,dv].
 *   alpha_mode        PDN_ALPHA_*;  log_alpha fp32, natural log of alpha, <= 0:
 *                     [B,H,T] (SCALAR) or [B,H,T,dk] (VEC); NULL for NONE.
 *                     The scalar-decay bf16 path (bf16 q/k/v, dk == 128,
 *                     scalar or no decay, scalar beta, symmetric keys, no
 *                     preconditioner) takes any value, floored at -80
 *                     (alpha = e^-80, below what an fp32 state resolves).
 *                     Every other prefill path clamps values below -10
 *                     (alpha < 4.5e-5) to -10.
 *   beta_mode         PDN_GATE_SCALAR [B,H,T] or PDN_GATE_VEC [B,H,T,dk]; fp32 >= 0.
 *   gamma_mode        PDN_GATE_SCALAR [B,H,T], PDN_GATE_VEC [B,H,T,dv] or
 *                     PDN_GAMMA_SAME_AS_BETA (gamma NULL; a VEC beta then needs
 *                     dk == dv); fp32 >= 0.
 *   key_mode          PDN_KEY_* (0 = symmetric, the default).
 *   precond_eps       < 0: preconditioner off.  >= 0: on, with this epsilon.
 *   precond_mode      PDN_PRECOND_INVERSE (0) or PDN_PRECOND_STABILISED (1).
 *   precond_x         stabilised mode: the bound x, 1 < x <= 2 (the pages use 1.5).
 *   precond_A0        [B,H,dk] fp32 start of the running k(.)k sum; NULL = zeros.
 *   precond_AT        [B,H,dk] fp32 running sum after token T; NULL = not written.
 *   S0                [B,H,dk,dv] fp32 initial state; NULL = zeros.
 *   ST                [B,H,dk,dv] fp32 final state; NULL = not written.
 *                     S0 == ST (in place) is allowed; no other aliasing is.
 *   o                 [B,H,T,dv] output in o_dtype.
 *   workspace, workspace_bytes   caller-owned device scratch of at least
 *                     pdn_chunk_fwd_workspace_size() bytes (may be 0 / NULL).
 */
typedef struct pdn_chunk_fwd_args {
    int32_t B, H, T, dk, dv;
    int32_t qkv_dtype;
    int32_t o_dtype;
    const void *q;
    const void *k;
    const void *v;
    int32_t alpha_mode;
    const float *log_alpha;
    int32_t beta_mode;
    const float *beta;
    int32_t gamma_mode;
    const float *gamma;
    int32_t key_mode;
    float precond_eps;
    int32_t precond_mode;
    float precond_x;
    const float *precond_A0;
    float *precond_AT;
    const float *S0;
    float *ST;
    void *o;
    void *workspace;
    size_t workspace_bytes;
} pdn_chunk_fwd_args;

/*
 * One decode step for every (b,h) against a resident fp32 state, in place.
 *
 *   B, H, dk, dv      sizes; B, H >= 1; dk, dv in {64, 128}.
 *   qkv_dtype         PDN_F32 or PDN_BF16;  q, k: [B,H,dk];  v: [B,H,dv].
 *   o_dtype           PDN_F32 or PDN_BF16;  o: [B,H,dv].
 *   alpha_mode, log_alpha ([B,H] or [B,H,dk]), beta_mode, beta ([B,H] or
 *   [B,H,dk]), gamma_mode, gamma ([B,H] or [B,H,dv]): as for the prefill with
 *   T == 1 (no clamp on log_alpha here).  key_mode as for the prefill.
 *   precond_eps       < 0 off; >= 0 on, and then precond_A ([B,H,dk] fp32) is
 *                     read, advanced by k(.)k and written back in place.
 *   precond_mode, precond_x  as for the prefill (every shape takes both modes).
 *   S                 [B,H,dk,dv] fp32, read and overwritten with S_t; 16-byte
 *                     aligned.
 */
typedef struct pdn_decode_args {
    int32_t B, H, dk, dv;
    int32_t qkv_dtype;
    int32_t o_dtype;
    const void *q;
    const void *k;
    const void *v;
    int32_t alpha_mode;
    const float *log_alpha;
    int32_t beta_mode;
    const float *beta;
    int32_t gamma_mode;
    const float *gamma;
    int32_t key_mode;
    float precond_eps;
    int32_t precond_mode;
    float precond_x;
    float *precond_A;
    float *S;
    void *o;
} pdn_decode_args;

/*
 * Backward of the prefill: gradients of
 *
 *   L = sum_{b,h,t} <dO_t, o_t> + sum_{b,h} <dST, S_T>
 *
 * with respect to q, k, v, log_alpha, beta, gamma, S0 and precond_A0 (the
 * gate-aware backward of "Gated DeltaNet-2", section 3 on chunkwise training:
 * with per-channel gates the decay cannot be pulled out of the dot products,
 * so the backward differentiates through the gate-scaled operands).  The forward is recomputed inside the call; nothing from a
 * previous pdn_chunk_fwd is needed.
 *
 *   fwd               the forward's arguments: sizes, q, k, v, gates, key_mode,
 *                     preconditioner (both modes), precond_A0, S0.  Its
 *                     o, ST, precond_AT, workspace and workspace_bytes are
 *                     ignored.  q/k/v fp32 or bf16; dk in {64, 128}; dv a
 *                     multiple of 32 and <= 256.  log_alpha is clamped at -10
 *                     as in the forward, and its gradient is zero where clamped.
 *   dO                [B,H,T,dv] fp32.          dST: [B,H,dk,dv] fp32, NULL = 0.
 *   dq, dk            [B,H,T,dk] fp32.          dv:  [B,H,T,dv] fp32.
 *   dlog_alpha        shape of log_alpha; NULL exactly when alpha_mode is NONE.
 *   dbeta             shape of beta.
 *   dgamma            shape of gamma; NULL exactly when gamma is "same as beta"
 *                     (that gradient is added into dbeta).
 *   dS0               [B,H,dk,dv] fp32; NULL = not written.
 *   dA0               [B,H,dk] fp32 (preconditioner on); NULL = not written.
 *   workspace, workspace_bytes   caller-owned device scratch of at least
 *                     pdn_chunk_bwd_workspace_size() bytes.
 * Every pointer 16-byte aligned; outputs must not overlap inputs or each
 * other.  In the symmetric key mode the gradient of sqrt(beta') is unbounded
 * at beta' = 0 (likewise gamma): such tokens give inf or NaN gradients.
 */
typedef struct pdn_chunk_bwd_args {
    pdn_chunk_fwd_args fwd;
    const float *dO;
    const float *dST;
    float *dq;
    float *dk;
    float *dv;
    float *dlog_alpha;
    float *dbeta;
    float *dgamma;
    float *dS0;
    float *dA0;
    void *workspace;
    size_t workspace_bytes;
} pdn_chunk_bwd_args;

/* PDN_ABI_VERSION of the loaded library. */
int pdn_abi_version(void);

/* Static, human-readable text for a PDN_* return code (never NULL). */
const char *pdn_strerror(int code);

/* Device scratch bytes pdn_chunk_fwd needs for these arguments (0 is valid).
 * Returns PDN_OK and writes *bytes, or a PDN_E* code for invalid arguments
 * (an int status with the size through a pointer, rather than a bare size_t
 * return, so that invalid arguments are reported as on every other call; a
 * size of 0 is a valid answer and cannot double as an error value).
 * Non-zero in two cases:
 *  - bf16 q/k/v with dk == 128 and a per-channel gate, the preconditioner or
 *    asymmetric keys: those calls first write, for every (b, h) and 32-token
 *    chunk, a 56 KiB record of gate-scaled operands and solve blocks (plus 512
 *    bytes of k(.)k sums with the preconditioner), which the state-carrying
 *    kernel then reads once;
 *  - few heads with long sequences and fp32 output (either gating): the
 *    sequence is then split into segments that run side by side, from their
 *    transitions and end states (fp32 [B,H,T,dk] plus a few
 *    [B,H,segments,dk,dv|dk] arrays).
 * The workspace holds no state between calls. */
int pdn_chunk_fwd_workspace_size(const pdn_chunk_fwd_args *args, size_t *bytes);

/* Validate only (no HIP call, no launch): PDN_OK or the code pdn_chunk_fwd
 * would return for these arguments before launching. */
int pdn_chunk_fwd_check(const pdn_chunk_fwd_args *args);

/* Prefill: o, and ST / precond_AT when given, for the recurrence at the top
 * of this file, computed chunkwise: per chunk the decayed Gram blocks of the
 * gain-scaled keys, a unit-lower-triangular (I + T)^-1 solve for the WY
 * factors, and a state carried from chunk to chunk ("Gated DeltaNet-2",
 * method section 3: the decay absorbed into the erase and write matrices, the
 * WY / UT form; "FG^2-GDN" section 2.3: the chunked form with fine-grained
 * gates).  Chunk length 64 (32 for the per-channel-gate path above); T need
 * not be a multiple of it and results do not depend on where chunks fall.
 * Returns PDN_OK, or a PDN_E* code before any launch (see the conventions);
 * PDN_EHIP if a launch fails. */
int pdn_chunk_fwd(const pdn_chunk_fwd_args *args, void *stream);

/* Validate only, as pdn_chunk_fwd_check. */
int pdn_decode_check(const pdn_decode_args *args);

/* Decode one token for all (b,h): the recurrence at the top of this file
 * with T = 1 against the resident state ("Gated DeltaNet-2", method section 1:
 * S_t = (I - k k^T) D_t S_{t-1} + k v^T with D_t = Diag(alpha_t), in the
 * gain placement of "FG^2-GDN" section 2.1; the running k (.) k of
 * "Preconditioned DeltaNet" section 2.2 advanced by one token).  Writes o,
 * overwrites S with S_t and precond_A with A_t; one pass over S.  Returns
 * PDN_OK, or a PDN_E* code before any launch; PDN_EHIP if the launch fails. */
int pdn_decode_step(const pdn_decode_args *args, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): pdn_chunk_fwd
 * with the scratch taken from a static device array of the library instead of
 * args->workspace (ignored here; may be NULL).  The array holds
 * PDN_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, from the first
 * call on that device until the process ends.  Calls that need more than that
 * (pdn_chunk_fwd_workspace_size() > PDN_NOALLOC_SCRATCH_BYTES) return
 * PDN_ESCRATCH before any launch: pass a workspace to pdn_chunk_fwd instead.
 * The call itself allocates nothing (no hipMalloc, no library allocation).
 * Every call on one GPU shares that GPU's array, and its contents persist
 * from call to call: calls on one GPU that overlap (on different streams or
 * from different threads without ordering) race on it and must not be made.
 * Inputs, outputs and return codes are those of pdn_chunk_fwd. */
#define PDN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int pdn_chunk_fwd_noalloc(const pdn_chunk_fwd_args *args, void *stream);

/* Device scratch bytes pdn_chunk_bwd needs (PDN_OK and *bytes, or a PDN_E*
 * code).  Per (b, h) and 32-token chunk: the chunk's gate-scaled operands and
 * solve blocks, its start state and the gradient of its end state
 * (dk x dv fp32 each), and dq/dk-side intermediates: about 9 KB per
 * token-head at dk = dv = 128.  The workspace holds no state between calls. */
int pdn_chunk_bwd_workspace_size(const pdn_chunk_bwd_args *args, size_t *bytes);

/* Validate only (no HIP call, no launch). */
int pdn_chunk_bwd_check(const pdn_chunk_bwd_args *args);

/* Backward of the prefill: every gradient listed above, asynchronously on
 * `stream`.  Chunk length 32; T need not be a multiple of it. */
int pdn_chunk_bwd(const pdn_chunk_bwd_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PDN_H */
