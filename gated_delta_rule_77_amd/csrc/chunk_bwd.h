// Backward of the chunked gated delta rule on gfx950 (device code, shared by
// chunk_bwd.hip and chunk_bwd_ilp.hip; not a public header): gradients of
// L = sum <dO, o> + <dST, S_T> with respect to q, k, v, the decay, the gains,
// S0 and A0 ("Gated DeltaNet-2", section 3: with per-channel gates the decay
// stays inside the dot products, so the backward differentiates through the
// gate-scaled operands).
//
// Per (b, h) and 32-token chunk, with G_r the in-chunk cumulative log decay
// (per channel), kr / kw the read / write keys and vw the written value of
// the key mode, Kg = kr (.) e^G, Qg = q (.) e^G, Kd = kw (.) e^(G_C - G),
// T_rs = sum_i kr_ri kw_si e^(G_ri - G_si) (s < r),
// P_rs = sum_i q_ri kw_si e^(G_ri - G_si) (s <= r), M = (I + T)^-1:
//
//   forward   X = Vw - Kg S,  U = M X,  O = Qg S + P U,  S' = Diag(e^G_C) S + Kd^T U
//   backward  Z = M^T (P^T dO + Kd dS'),
//             dS = Diag(e^G_C) dS' + Qg^T dO - Kg^T Z,
//             dQg = dO S^T, dKg = -Z S^T, dKd = U dS'^T, dVw = Z,
//             dP = dO U^T (s <= r), dT = -Z U^T (s < r), dGamma_C = rowsum(S (.) dS')
//
// and from those to q, k, v and the gates through the pairwise decays.
//
// Kernels, in launch order:
//   bwd_ksum / bwd_scan    preconditioner: running k (.) k before each chunk
//   bwd_prep               per chunk: Kg, Qg, Kd, Vw, M, P, e^G_C (the record)
//   bwd_states             per (b, h, 32 value columns), both passes side by
//                          side: chunks in order (the chunk start states S
//                          and U) and in reverse (dS' per chunk, Z, dS0)
//   bwd_grads              per chunk: the dv contractions (dQg, dKg, dKd, dP,
//                          dT, dGamma_C), fp32 16x16x4 MFMAs, then
//                          the pairwise sums (MFMA) and dq, dk, dv, d log alpha,
//                          dbeta, dgamma, and the preconditioner's dA
//   bwd_scan (reverse) / bwd_dA_apply   preconditioner: dk += 2 k (.) sum_{s>=t} dA_s
//
// Every product is an fp32 MFMA (exact fp32 products, fp32 accumulation) or
// fp32 VALU.  The pairwise decays e^(G_r - G_s) inside a chunk enter the MFMA
// products split at a reference row (the middle of each 16-token block, or
// the block boundary), which the clamp of log alpha at -10 keeps within the
// fp32 range; the gradient of log alpha is zero where the clamp acts.
#pragma once
#include "common.h"
#include "kernels.h"

namespace pdn {

struct BwdParams {
    int T, dv, nc;
    long nbh;
    const void* q;
    const void* k;
    const void* v;
    int amode, bmode, gmode, kmode;
    const float* la;
    const float* beta;
    const float* gamma;
    float eps;
    int pre;
    int stab;   // stabilised preconditioner coefficient x^-(r / (1 + |r|))
    float lnx;  // ln x of that coefficient
    const float* A0;
    const float* S0;
    const float* dO;
    const float* dST;
    float* dq;
    float* dk;
    float* dvo;
    float* dla;
    float* dbeta;
    float* dgamma;
    float* dS0;
    float* dA0;
    // workspace
    float* rec;    // [BH][nc][REC]
    float* st;     // [BH][nc+1][DK][dv] chunk start states (entry nc: S_T)
    float* dst;    // [BH][nc][DK][dv] gradient of each chunk's end state
    float* U;      // [BH][nc*BC][dv]
    float* Z;      // [BH][nc*BC][dv]
    float* dgr;    // [BH][nc][DGR]
    float* apre;   // [BH][nc][DK] running k (.) k before each chunk (with A0)
    float* ksum;   // [BH][nc][DK] per-chunk k (.) k sums
    float* dAin;   // [BH][nc*BC][DK] in-chunk suffix sums of dA
    float* dAc;    // [BH][nc][DK] chunk totals of dA
    float* dAsuf;  // [BH][nc][DK] sums of dA over the later chunks
    float* mu;     // [BH][nc*BC] stabilised mode: channel mean of ln(A + eps) per token
};

// Launchers of the kernels that chunk_bwd_ilp.hip builds with the
// instruction-level-parallelism scheduler: the state passes on 32-column
// tiles and the gradient kernel (measured faster that way; the preparation
// kernel and the 16-column state passes are faster with the default
// scheduler and stay in chunk_bwd.hip).
template <int DK>
void launch_bwd_states_wide(const BwdParams& p, unsigned grid, long units, hipStream_t s);
template <int DK, bool BF16>
void launch_bwd_grads(const BwdParams& p, unsigned grid, hipStream_t s);

namespace {

constexpr int BC = 32;   // tokens per chunk
constexpr int NT = 256;  // threads per workgroup (four waves)
constexpr int JT = 32;   // value columns per state tile

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}



// record of one chunk: Kg, Qg, Kd [BC][DK]; Vw [BC][dv]; M, P [BC][BC]; e^G_C [DK]
template <int DK>
__host__ __device__ constexpr long rec_floats_fixed() { return 3L * BC * DK + 2L * BC * BC + DK; }
template <int DK>
__host__ __device__ inline long rec_floats(int dv) { return rec_floats_fixed<DK>() + static_cast<long>(BC) * dv; }
template <int DK>
__host__ __device__ inline long rec_vw(int) { return 3L * BC * DK; }
template <int DK>
__host__ __device__ inline long rec_m(int dv) { return 3L * BC * DK + static_cast<long>(BC) * dv; }
template <int DK>
__host__ __device__ inline long rec_p(int dv) { return rec_m<DK>(dv) + BC * BC; }
template <int DK>
__host__ __device__ inline long rec_gc(int dv) { return rec_p<DK>(dv) + BC * BC; }
// gradient record: dQg, dKg, dKd [BC][DK]; dP, dT [BC][BC]; dGamma_C [DK]
template <int DK>
__host__ __device__ constexpr long dgr_floats() { return 3L * BC * DK + DK; }

// ---------------------------------------------------------------------------
// per-token gates (shared by the prep and the gradient kernels)
// ---------------------------------------------------------------------------

// Per-token gate values.  Every load is unconditional (the token index is
// clamped to T - 1 and the mode picks a base pointer and stride), and the
// result is selected afterwards, so that a column's loads issue back to back.
__device__ __forceinline__ long tclamp(const BwdParams& p, long t) { return t < p.T ? t : p.T - 1; }

// raw log decay of token t, channel i (without decay: some valid element)
template <int DK>
__device__ __forceinline__ float tok_la_raw(const BwdParams& p, long bh, long t, int i) {
    const long tc = tclamp(p, t);
    const bool vec = p.amode == PDN_ALPHA_VEC;
    const float* base = p.amode == PDN_ALPHA_NONE ? p.beta : p.la;
    return base[vec ? (bh * p.T + tc) * DK + i : bh * p.T + tc];
}
// clamped natural-log decay of token t (0 beyond T or without decay)
template <int DK>
__device__ __forceinline__ float tok_la(const BwdParams& p, long bh, long t, int i) {
    const float x = tok_la_raw<DK>(p, bh, t, i);
    return (t < p.T && p.amode != PDN_ALPHA_NONE) ? fmaxf(x, kLogAlphaMin) : 0.f;
}
// raw erase gain (1 beyond T, so that padded rows carry finite zero gradients)
template <int DK>
__device__ __forceinline__ float tok_beta(const BwdParams& p, long bh, long t, int i) {
    const long tc = tclamp(p, t);
    const float x = p.beta[p.bmode == PDN_GATE_VEC ? (bh * p.T + tc) * DK + i : bh * p.T + tc];
    return t < p.T ? x : 1.f;
}
// raw value gain of column j (raw beta when gamma is "same as beta")
template <int DK>
__device__ __forceinline__ float tok_gamma(const BwdParams& p, long bh, long t, int j) {
    const long tc = tclamp(p, t);
    const bool same = p.gmode == PDN_GAMMA_SAME_AS_BETA;
    const bool vec = same ? p.bmode == PDN_GATE_VEC : p.gmode == PDN_GATE_VEC;
    const float* base = same ? p.beta : p.gamma;
    const long idx = vec ? (bh * p.T + tc) * (same ? DK : p.dv) + j : bh * p.T + tc;
    const float x = base[idx];
    return t < p.T ? x : 1.f;
}
// q / k / v element (0 beyond T)
template <bool BF16>
__device__ __forceinline__ float tok_in(const BwdParams& p, const void* x, long bh, long t, int w, int i) {
    const float v = load_in<BF16>(x, (bh * p.T + tclamp(p, t)) * w + i);
    return t < p.T ? v : 0.f;
}

// write key, read key of one channel from k and the erase gain b
__device__ __forceinline__ void keys_of(int kmode, float b, float kk, float& kw, float& kr) {
    if (kmode == PDN_KEY_SYMMETRIC) {
        kw = sqrtf(b) * kk;
        kr = kw;
    } else if (kmode == PDN_KEY_ERASE_GATE) {
        kw = kk;
        kr = b * kk;
    } else {
        kw = b * kk;
        kr = kk;
    }
}
// value scale of a mode: vw = scale * v
__device__ __forceinline__ float value_scale(int kmode, int gmode, float g) {
    if (kmode == PDN_KEY_SYMMETRIC) return sqrtf(g);
    if (kmode == PDN_KEY_WRITE_GATE && gmode == PDN_GAMMA_SAME_AS_BETA) return 1.f;
    return g;
}
// d vw / d g divided by v
__device__ __forceinline__ float value_dscale(int kmode, int gmode, float g) {
    if (kmode == PDN_KEY_SYMMETRIC) return 0.5f / sqrtf(g);
    if (kmode == PDN_KEY_WRITE_GATE && gmode == PDN_GAMMA_SAME_AS_BETA) return 0.f;
    return 1.f;
}

// Per-thread views of one key channel's per-token inputs over a chunk: base
// pointers and strides are fixed once; a row index beyond T is clamped (the
// value is then masked by the caller).
template <int DK, bool BF16>
struct ColView {
    const void* k;
    const void* q;
    const float* la;
    const float* be;
    long kq_row, la_row, be_row;  // element strides per token
    int rmax;                     // last valid row of the chunk
    __device__ ColView(const BwdParams& p, long bh, long t0, int i) {
        const long tok0 = bh * p.T + t0;
        rmax = static_cast<int>(min(static_cast<long>(BC - 1), p.T - 1 - t0));
        const size_t esz = BF16 ? 2 : 4;
        k = static_cast<const char*>(p.k) + (tok0 * DK + i) * esz;
        q = static_cast<const char*>(p.q) + (tok0 * DK + i) * esz;
        kq_row = DK;
        const bool lav = p.amode == PDN_ALPHA_VEC;
        la = (p.amode == PDN_ALPHA_NONE ? p.beta + tok0 : p.la + (lav ? tok0 * DK + i : tok0));
        la_row = lav ? DK : 1;
        const bool bv = p.bmode == PDN_GATE_VEC;
        be = p.beta + (bv ? tok0 * DK + i : tok0);
        be_row = bv ? DK : 1;
    }
    __device__ __forceinline__ int rc(int r) const { return r < rmax ? r : rmax; }
    __device__ __forceinline__ float kv(int r) const { return load_in<BF16>(k, rc(r) * kq_row); }
    __device__ __forceinline__ float qv(int r) const { return load_in<BF16>(q, rc(r) * kq_row); }
    __device__ __forceinline__ float lav(int r) const { return la[rc(r) * la_row]; }
    __device__ __forceinline__ float bev(int r) const { return be[rc(r) * be_row]; }
};

// ---------------------------------------------------------------------------
// preconditioner: A before each chunk
// ---------------------------------------------------------------------------
template <int DK, bool BF16>
__global__ void __launch_bounds__(DK) bwd_ksum_kernel(BwdParams p) {
    const long bh = blockIdx.x / p.nc;
    const long c = blockIdx.x % p.nc;
    const int i = threadIdx.x;
    // every row loaded (clamped) before any is used, rows past T masked after
    float kk[BC];
#pragma unroll
    for (int r = 0; r < BC; ++r) kk[r] = load_in<BF16>(p.k, (bh * p.T + tclamp(p, c * BC + r)) * DK + i);
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < BC; ++r) {
        const float x = c * BC + r < p.T ? kk[r] : 0.f;
        s += x * x;
    }
    p.ksum[(bh * p.nc + c) * DK + i] = s;
}

// Exclusive running sum over the chunks of each (b, h) and channel, forward
// (out[c] = init + sum of in[c'] for c' < c) or reverse (REV: the sum over
// c' > c), with the grand total (init + every chunk) written to `total` if
// given.  One workgroup per (b, h, 32 channels): thread (segment, channel)
// sums a run of chunks, the segment totals are prefixed through LDS, and a
// second pass writes.  Each run is a chain of dependent loads, so the runs
// are kept short (32 segments per head).
constexpr int SCAN_SEG = 32;
constexpr int SCAN_CH = 32;
template <int DK, bool REV>
__global__ void __launch_bounds__(SCAN_SEG * SCAN_CH) bwd_scan_kernel(const float* in, float* out, const float* init,
                                                                      float* total, long nc) {
    static_assert(DK % SCAN_CH == 0, "whole channel groups");
    __shared__ float tot[SCAN_SEG][SCAN_CH];
    const long bh = blockIdx.x / (DK / SCAN_CH);
    const int ci = threadIdx.x % SCAN_CH;
    const int i = static_cast<int>(blockIdx.x % (DK / SCAN_CH)) * SCAN_CH + ci;
    const int sg = threadIdx.x / SCAN_CH;
    const long len = (nc + SCAN_SEG - 1) / SCAN_SEG;
    const long q0 = min(sg * len, nc), q1 = min(q0 + len, nc);  // positions in scan order
    auto at = [&](long q) { return (bh * nc + (REV ? nc - 1 - q : q)) * DK + i; };
    float sum = 0.f;
    long q = q0;
    for (; q + 8 <= q1; q += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = in[at(q + u)];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; q < q1; ++q) sum += in[at(q)];
    tot[sg][ci] = sum;
    __syncthreads();
    float run = init ? init[bh * DK + i] : 0.f;
    for (int s2 = 0; s2 < sg; ++s2) run += tot[s2][ci];
    q = q0;
    for (; q + 8 <= q1; q += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = in[at(q + u)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            out[at(q + u)] = run;
            run += v[u];
        }
    }
    for (; q < q1; ++q) {
        const float v = in[at(q)];
        out[at(q)] = run;
        run += v;
    }
    if (total && sg == SCAN_SEG - 1) total[bh * DK + i] = run;
}

// ---------------------------------------------------------------------------
// per-chunk record
// ---------------------------------------------------------------------------
// T and P as fp32 MFMA products over the key channels: with the decay split
// at the middle row m_b of each 16-token block (L_r = e^(G_r - G_mb),
// R_s = e^(G_mb - G_s), L_r R_s = e^(G_r - G_s) inside a block, both factors
// within e^(+-80) by the clamp on log alpha), T_rs = sum_i (kr L)_ri (kw R)_si
// and P_rs = sum_i (q L)_ri (kw R)_si on the two diagonal 16 x 16 blocks; the
// block below the diagonal uses (kw R c)_s with c = e^(G_24 - G_8), since
// e^(G_r - G_s) = L_r c R_s there.
template <int DK, bool BF16, bool STAB>
__global__ void __launch_bounds__(NT, 3) bwd_prep_kernel(BwdParams p) {
    // 51 KB of LDS, so that three workgroups share a CU
    constexpr int LS = DK + 4;  // read as [row][k]; the 4 pad columns hold scalars
    __shared__ float sKrL[BC][LS];  // after the products: T
    __shared__ float sQL[BC][LS];   // pad column DK: the mean of ln(A + eps) per row
    __shared__ float sKwR[BC][LS];  // before the operands: the per-part sums; pad: c per channel
    const long bh = blockIdx.x / p.nc;
    const long c = blockIdx.x % p.nc;
    const long t0 = c * BC;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    float* R = p.rec + (bh * p.nc + c) * rec_floats<DK>(p.dv);
    // thread (channel i, part h) owns rows h RPT .. h RPT + RPT - 1 of channel i;
    // the scans cross the parts through LDS
    constexpr int NH = NT / DK, RPT = BC / NH;
    static_assert(NH * 2 * DK <= BC * LS && BC * (BC + 1) <= BC * LS && DK <= 4 * BC,
                  "the aliased scratch fits its buffer");
    // per-part sums of the log decay and of k (.) k
    float(*sPart)[2][DK] = reinterpret_cast<float(*)[2][DK]>(&sKwR[0][0]);
    float(*sT)[BC + 1] = reinterpret_cast<float(*)[BC + 1]>(&sKrL[0][0]);
    __shared__ float sRef[3][DK];       // G at rows 8, 24 and 31 of each channel
    const int i = tid % DK, h = tid / DK, r0 = h * RPT;
    const ColView<DK, BF16> cv(p, bh, t0, i);
    const bool has_decay = p.amode != PDN_ALPHA_NONE;
    // The value tile Vw = v (.) scale(gamma), in items of 8 consecutive
    // columns of one row (items past the tile reread item 0, rows past T
    // reread row T - 1; both are masked when written).  With bf16 inputs the
    // loads are issued first of all, so that their round trip overlaps the
    // scans below; the other instantiations have no registers to spare for
    // that and issue them where the tile is written.
    constexpr int MAXI = BC * 256 / 8 / NT;  // dv <= 256
    constexpr bool kEarly = BF16 && !STAB;
    const int nit = BC * p.dv / 8;
    const bool gsame = p.gmode == PDN_GAMMA_SAME_AS_BETA;
    const bool gvec = gsame ? p.bmode == PDN_GATE_VEC : p.gmode == PDN_GATE_VEC;
    const float* gbase = gsame ? p.beta : p.gamma;
    const int gw = gsame ? DK : p.dv;
    f32x4 vv[MAXI][2], gv[MAXI][2];
    auto load_v = [&]() {
#pragma unroll
    for (int m = 0; m < MAXI; ++m) {
        const int it = tid + m * NT < nit ? tid + m * NT : 0;
        const int r = it / (p.dv / 8), j = 8 * (it % (p.dv / 8));
        const long tc = bh * p.T + tclamp(p, t0 + r);
        if constexpr (BF16) {
            const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) + tc * p.dv + j);
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vv[m][e >> 1][2 * (e & 1)] = __uint_as_float(w4[e] << 16);
                vv[m][e >> 1][2 * (e & 1) + 1] = __uint_as_float(w4[e] & 0xffff0000u);
            }
        } else {
            const float* src = static_cast<const float*>(p.v) + tc * p.dv + j;
            vv[m][0] = *reinterpret_cast<const f32x4*>(src);
            vv[m][1] = *reinterpret_cast<const f32x4*>(src + 4);
        }
        if (gvec) {
            gv[m][0] = *reinterpret_cast<const f32x4*>(gbase + tc * gw + j);
            gv[m][1] = *reinterpret_cast<const f32x4*>(gbase + tc * gw + j + 4);
        } else {
            const float x = gbase[tc];
            gv[m][0] = f32x4{x, x, x, x};
            gv[m][1] = gv[m][0];
        }
    }
    };
    if constexpr (kEarly) load_v();
    // every load of the own rows first
    float kk[RPT], qq[RPT], g[RPT], bb[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        kk[u] = cv.kv(r0 + u);
        qq[u] = cv.qv(r0 + u);
        g[u] = cv.lav(r0 + u);
        bb[u] = cv.bev(r0 + u);
    }
    float gs = 0.f, as = 0.f;
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const bool valid = t0 + r0 + u < p.T;
        g[u] = (valid && has_decay) ? fmaxf(g[u], kLogAlphaMin) : 0.f;
        if (!valid) {
            kk[u] = 0.f;
            qq[u] = 0.f;
            bb[u] = 1.f;
        }
        gs += g[u];
        as += kk[u] * kk[u];
    }
    sPart[h][0][i] = gs;
    sPart[h][1][i] = as;
    __syncthreads();
    float Gin = 0.f, Ain = p.pre ? p.apre[(bh * p.nc + c) * DK + i] : 0.f;
    for (int h2 = 0; h2 < h; ++h2) {
        Gin += sPart[h2][0][i];
        Ain += sPart[h2][1][i];
    }
    {
        float run = Gin;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            run += g[u];
            g[u] = run;
            const int r = r0 + u;
            if (r == 8) sRef[0][i] = run;
            if (r == 24) sRef[1][i] = run;
            if (r == BC - 1) sRef[2][i] = run;
        }
    }
    if constexpr (STAB) {
        // the channel mean of ln(A + eps) per token (sKrL holds ln(A + eps) for now)
        float A = Ain;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            A += kk[u] * kk[u];
            sKrL[r0 + u][i] = logf(A + p.eps);
        }
        __syncthreads();
        if (tid < BC) {
            float m = 0.f;
            for (int ii = 0; ii < DK; ++ii) m += sKrL[tid][ii];
            m *= 1.f / DK;
            sQL[tid][DK] = m;
            p.mu[bh * static_cast<long>(p.nc) * BC + t0 + tid] = m;
        }
    }
    __syncthreads();
    {
        const float g8 = sRef[0][i], g24 = sRef[1][i], gc = sRef[2][i];
        const float cst = __expf(g24 - g8);
        float A = Ain;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int r = r0 + u;
            float b = bb[u];
            if (p.pre) {
                A += kk[u] * kk[u];
                if constexpr (STAB) {
                    const float x = logf(A + p.eps) - sQL[r][DK];
                    b = b * __expf(-(x / (1.f + fabsf(x))) * p.lnx);
                } else {
                    b = b / (A + p.eps);
                }
            }
            float kw, kr;
            keys_of(p.kmode, b, kk[u], kw, kr);
            const float e = __expf(g[u]);
            R[r * DK + i] = kr * e;
            R[BC * DK + r * DK + i] = qq[u] * e;
            R[2 * BC * DK + r * DK + i] = kw * __expf(gc - g[u]);
            const float gm = r < 16 ? g8 : g24;
            const float L = __expf(g[u] - gm), Rs = __expf(gm - g[u]);
            sKrL[r][i] = kr * L;
            sQL[r][i] = qq[u] * L;
            sKwR[r][i] = kw * Rs;
        }
        if (h == 0) {
            R[rec_gc<DK>(p.dv) + i] = __expf(gc);
            sKwR[i / 4][DK + i % 4] = cst;
        }
    }
    float* Rvw = R + rec_vw<DK>(p.dv);
    if constexpr (!kEarly) load_v();
#pragma unroll
    for (int m = 0; m < MAXI; ++m) {
        const int it = tid + m * NT;
        const int r = it / (p.dv / 8), j = 8 * (it % (p.dv / 8));
        const bool live = t0 + r < p.T;
        if (it < nit)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = live ? vv[m][hh][e] * value_scale(p.kmode, p.gmode, gv[m][hh][e]) : 0.f;
                *reinterpret_cast<f32x4*>(Rvw + r * p.dv + j + 4 * hh) = o;
            }
    }
    __syncthreads();
    // six 16 x 16 tiles: T (0,0), (1,1), (1,0) and P likewise; wave w takes
    // tile w and, for w < 2, tile w + 4
    float* Rp = R + rec_p<DK>(p.dv);
    f32x4 accT = {0.f, 0.f, 0.f, 0.f};  // the T tile of waves 0..2
    for (int tile = w; tile < 6; tile += 4) {
        const bool isP = tile >= 3;
        const int which = tile % 3;  // 0: (0,0), 1: (1,1), 2: (1,0)
        const int rb = which == 0 ? 0 : 1, sb = which == 1 ? 1 : 0;
        const float(*Aop)[LS] = isP ? sQL : sKrL;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (which == 2) {
            // across the blocks: the kw R rows of block 0 times c of the channel
#pragma unroll 8
            for (int k = 0; k < DK; k += 4)
                acc = mfma4(Aop[16 + ln][k + g4], sKwR[ln][k + g4] * sKwR[k / 4][DK + g4], acc);
        } else {
#pragma unroll 8
            for (int k = 0; k < DK; k += 4)
                acc = mfma4(Aop[16 * rb + ln][k + g4], sKwR[16 * sb + ln][k + g4], acc);
        }
        if (isP) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e, s2 = 16 * sb + ln;
                Rp[r * BC + s2] = s2 <= r ? acc[e] : 0.f;
            }
        } else {
            accT = acc;
        }
    }
    for (int idx = tid; idx < 16 * 16; idx += NT) Rp[(idx / 16) * BC + 16 + idx % 16] = 0.f;
    __syncthreads();  // every wave is done with the operands: sKrL takes T
    if (w < 3) {
        const int rb = w == 0 ? 0 : 1, sb = w == 1 ? 1 : 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e, s2 = 16 * sb + ln;
            sT[r][s2] = s2 < r ? accT[e] : 0.f;
        }
    }
    // the upper-right block is zero
    for (int idx = tid; idx < 16 * 16; idx += NT) sT[idx / 16][16 + idx % 16] = 0.f;
    __syncthreads();
    // M = (I + T)^-1, one column per thread: x_r = [r == j] - sum_{s<r} T_rs x_s
    float* Rm = R + rec_m<DK>(p.dv);
    if (tid < BC) {
        // column j in registers; T rows are broadcast reads (x_s = 0 for s < j)
        const int j = tid;
        float x[BC];
#pragma unroll
        for (int r = 0; r < BC; ++r) {
            float acc = r == j ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < r; ++s2) acc -= sT[r][s2] * x[s2];
            x[r] = r < j ? 0.f : acc;
            Rm[r * BC + j] = x[r];
        }
    }
}

// ---------------------------------------------------------------------------
// state passes: one workgroup per (b, h, 32 value columns); state tile
// DK x 32 in MFMA accumulators, (DK / 16) x 2 tiles of 16 x 16 over 4 waves.
// ---------------------------------------------------------------------------
// staged copy of [rows][W] floats (W % 4 == 0, rows * W / 4 == n4) from
// global to registers and from registers to an LDS array with row stride LS
template <int W, int N4>
struct Tile4 {
    static constexpr int PER = (N4 + NT - 1) / NT;
    f32x4 v[PER];
    // every thread loads (past the tile it rereads a valid element that it
    // then does not store): a load on one path only would make the compiler
    // wait for all outstanding loads where the paths join
    __device__ __forceinline__ void load(const float* g, long gstride) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int idx = (N4 % NT == 0 || tid + u * NT < N4) ? tid + u * NT : (tid + u * NT) % N4;
            const int r = idx / (W / 4), c4 = idx % (W / 4);
            v[u] = *reinterpret_cast<const f32x4*>(g + r * gstride + 4 * c4);
        }
    }
    template <int LS>
    __device__ __forceinline__ void store(float* l) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int idx = tid + u * NT;
            if (N4 % NT == 0 || idx < N4) {
                const int r = idx / (W / 4), c4 = idx % (W / 4);
                *reinterpret_cast<f32x4*>(l + r * LS + 4 * c4) = v[u];
            }
        }
    }
};

// Scheduling hint for the block just emitted: the LDS operand reads run a few
// MFMAs ahead, and every M MFMAs are followed by one global load (N of them)
// and the next reads, so that the next chunk's loads issue one at a time
// between the MFMAs instead of in one burst ahead of them (a burst of ~30 1 KiB
// loads per wave keeps the CU's address unit busy for ~1,000-2,000 cycles,
// during which the wave issues nothing else).
template <int N, int M = 1>
__device__ __forceinline__ void interleave_loads() {
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // global load
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * M, 0);  // LDS reads
    }
}

// (b, h) and first value column of state-pass unit u.  Both workgroups of a
// unit run on XCD u mod kXcds (see bwd_states_kernel); when the head count
// allows, all column tiles of a head get the same u mod kXcds, so that they
// share the chunk records in that XCD's L2.
template <int SJ>
__device__ __forceinline__ void unit_tile(const BwdParams& p, long u, long& bh, int& j0) {
    const int ntile = p.dv / SJ;
    if (p.nbh % kXcds == 0) {
        bh = (u / (static_cast<long>(kXcds) * ntile)) * kXcds + u % kXcds;
        j0 = static_cast<int>((u / kXcds) % ntile) * SJ;
    } else {
        bh = u / ntile;
        j0 = static_cast<int>(u % ntile) * SJ;
    }
}

// LDS of the forward state pass, in floats (SJ value columns per workgroup)
template <int DK, int SJ>
constexpr int fwd_lds_floats() {
    return BC * (DK + 4) + BC * (DK + 16) + BC * (BC + 4) + 2 * BC * (SJ + 16) + DK * (SJ + 16) + DK;
}

// Tile assignment of the state passes (SJ = 32 or 16 value columns per
// workgroup, four waves): the BC x SJ tiles of X / U (forward) and Y / Z
// (reverse) go one per wave (with SJ = 16, waves 2 and 3 have none and only
// take part in the barriers); the DK x SJ state tile is NSB 16 x 16 blocks per
// wave.  Narrow tiles double the workgroups of a call, for few heads.
template <int DK, int SJ>
struct StateTiles {
    static constexpr int CB = SJ / 16;              // 16-column blocks
    static constexpr int NSB = DK / 16 * CB / 4;    // state blocks per wave
    static constexpr int NXT = BC / 16 * CB;        // waves with an X / Y tile
    static __device__ __forceinline__ int rb(int w) { return CB == 2 ? w >> 1 : w & 1; }
    static __device__ __forceinline__ int xcb(int w) { return CB == 2 ? w & 1 : 0; }
    static __device__ __forceinline__ int sib(int q) { return q / CB; }   // state block q: row block
    static __device__ __forceinline__ int scb(int q) { return q % CB; }   // and column block
};

// This wave's blocks of a DK x SJ state tile (a null source gives zeros): one
// branch around all the loads, so that they are issued together (a per-element
// test would make the compiler wait for each load in turn).
template <int NSB, class ST>
__device__ __forceinline__ void load_state_tile(const float* src, long off, int dv, int w, f32x4 (&acc)[NSB]) {
    const int lane = threadIdx.x & 63, ln = lane & 15, g4 = lane >> 4;
    if (src) {
#pragma unroll
        for (int m = 0; m < NSB; ++m) {
            const int q = w * NSB + m, ib = ST::sib(q), cb = ST::scb(q);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[m][e] = src[off + (16 * ib + 4 * g4 + e) * dv + 16 * cb + ln];
        }
    } else {
#pragma unroll
        for (int m = 0; m < NSB; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// forward state pass of workgroup `unit` (b, h, SJ value columns)
template <int DK, int SJ>
__device__ __forceinline__ void state_fwd_body(const BwdParams& p, float* smem, long unit) {
    using ST = StateTiles<DK, SJ>;
    constexpr int NSB = ST::NSB;  // state tiles per wave
    // sKg read as [row][k] (stride 4 mod 64 banks); sKd read as [k][col] (stride 16 mod 64)
    float(*sKg)[DK + 4] = reinterpret_cast<float(*)[DK + 4]>(smem);
    float(*sKd)[DK + 16] = reinterpret_cast<float(*)[DK + 16]>(smem + BC * (DK + 4));
    float(*sM)[BC + 4] = reinterpret_cast<float(*)[BC + 4]>(smem + BC * (DK + 4) + BC * (DK + 16));
    float* base = smem + BC * (DK + 4) + BC * (DK + 16) + BC * (BC + 4);
    float(*sX)[SJ + 16] = reinterpret_cast<float(*)[SJ + 16]>(base);
    float(*sU)[SJ + 16] = reinterpret_cast<float(*)[SJ + 16]>(base + BC * (SJ + 16));
    float(*sS)[SJ + 16] = reinterpret_cast<float(*)[SJ + 16]>(base + 2 * BC * (SJ + 16));
    float* sGc = base + 2 * BC * (SJ + 16) + DK * (SJ + 16);
    long bh;
    int j0;
    unit_tile<SJ>(p, unit, bh, j0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    const long Tp = static_cast<long>(p.nc) * BC;
    const long SZ = static_cast<long>(DK) * p.dv;
    const long RF = rec_floats<DK>(p.dv);
    f32x4 sacc[NSB];
    load_state_tile<NSB, ST>(p.S0, bh * SZ + j0, p.dv, w, sacc);  // every load before any use
#pragma unroll
    for (int m = 0; m < NSB; ++m) {
        const int q = w * NSB + m, ib = ST::sib(q), cb = ST::scb(q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * ib + 4 * g4 + e, col = 16 * cb + ln;
            sS[row][col] = sacc[m][e];
            p.st[bh * (p.nc + 1) * SZ + row * p.dv + j0 + col] = sacc[m][e];
        }
    }
    // X / Y tile of this wave (SJ = 16: waves 2 and 3 compute the tiles of
    // waves 0 and 1 again, which keeps their loads and MFMAs on the same path,
    // and store nothing)
    const int rb = ST::rb(w), xcb = ST::xcb(w);
    const bool xown = w < ST::NXT;
    // the next chunk's operands, loaded while the current one is processed
    Tile4<DK, BC * DK / 4> nKg, nKd;
    Tile4<BC, BC * BC / 4> nM;
    Tile4<DK, DK / 4> nGc;
    float nVw[4];
    auto fetch = [&](long c) {
        const float* R = p.rec + (bh * p.nc + c) * RF;
        nKg.load(R, DK);
        nKd.load(R + 2 * BC * DK, DK);
        nM.load(R + rec_m<DK>(p.dv), BC);
        nGc.load(R + rec_gc<DK>(p.dv), DK);
        const float* Rvw = R + rec_vw<DK>(p.dv);
#pragma unroll
        for (int e = 0; e < 4; ++e) nVw[e] = Rvw[(16 * rb + 4 * g4 + e) * p.dv + j0 + 16 * xcb + ln];
    };
    fetch(0);
    for (long c = 0; c < p.nc; ++c) {
        __syncthreads();  // the previous chunk's LDS reads are done
        nKg.template store<DK + 4>(&sKg[0][0]);
        nKd.template store<DK + 16>(&sKd[0][0]);
        nM.template store<BC + 4>(&sM[0][0]);
        nGc.template store<DK>(&sGc[0]);
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = nVw[e];
        __syncthreads();
        // the next chunk's loads (the last chunk rereads itself, so that no
        // branch splits them from the MFMAs below)
        fetch(c + 1 < p.nc ? c + 1 : c);
        // X = Vw - Kg S: tile (rb, xcb)
#pragma unroll
        for (int k = 0; k < DK; k += 4) x = mfma4(-sKg[16 * rb + ln][k + g4], sS[k + g4][16 * xcb + ln], x);
        interleave_loads<DK / 4>();
        if (xown)
#pragma unroll
            for (int e = 0; e < 4; ++e) sX[16 * rb + 4 * g4 + e][16 * xcb + ln] = x[e];
        __syncthreads();
        // U = M X
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < BC; k += 4) u = mfma4(sM[16 * rb + ln][k + g4], sX[k + g4][16 * xcb + ln], u);
        if (xown)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e;
                sU[r][16 * xcb + ln] = u[e];
                p.U[(bh * Tp + c * BC + r) * p.dv + j0 + 16 * xcb + ln] = u[e];
            }
        __syncthreads();
        // S <- Diag(e^G_C) S + Kd^T U
#pragma unroll
        for (int m = 0; m < NSB; ++m) {
            const int q = w * NSB + m, ib = ST::sib(q), cb = ST::scb(q);
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc[m][e] *= sGc[16 * ib + 4 * g4 + e];
#pragma unroll
            for (int k = 0; k < BC; k += 4)
                sacc[m] = mfma4(sKd[k + g4][16 * ib + ln], sU[k + g4][16 * cb + ln], sacc[m]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * ib + 4 * g4 + e, col = 16 * cb + ln;
                sS[row][col] = sacc[m][e];
                p.st[(bh * (p.nc + 1) + c + 1) * SZ + row * p.dv + j0 + col] = sacc[m][e];
            }
        }
    }
}

// LDS of the reverse state pass, in floats.  M and P reach the MFMAs from
// registers, Z reuses Y's buffer, and the tiles use narrow row strides (some
// two-way bank conflicts), so that both passes fit on one CU together.
template <int DK, int SJ>
constexpr int bwd_lds_floats() {
    return 3 * BC * (DK + 4) + 2 * BC * (SJ + 4) + DK * (SJ + 4) + DK;
}

// reverse state pass of workgroup `unit` (b, h, SJ value columns)
template <int DK, int SJ>
__device__ __forceinline__ void state_bwd_body(const BwdParams& p, float* smem, long unit) {
    using ST = StateTiles<DK, SJ>;
    constexpr int NSB = ST::NSB;
    // sQg, sKg read as [k][col]; sKd as [row][k]
    float(*sQg)[DK + 4] = reinterpret_cast<float(*)[DK + 4]>(smem);
    float(*sKg)[DK + 4] = reinterpret_cast<float(*)[DK + 4]>(smem + BC * (DK + 4));
    float(*sKd)[DK + 4] = reinterpret_cast<float(*)[DK + 4]>(smem + 2 * BC * (DK + 4));
    float* base = smem + 3 * BC * (DK + 4);
    float(*sdO)[SJ + 4] = reinterpret_cast<float(*)[SJ + 4]>(base);
    float(*sY)[SJ + 4] = reinterpret_cast<float(*)[SJ + 4]>(base + BC * (SJ + 4));  // then Z
    float(*sdS)[SJ + 4] = reinterpret_cast<float(*)[SJ + 4]>(base + 2 * BC * (SJ + 4));
    float* sGc = base + 2 * BC * (SJ + 4) + DK * (SJ + 4);
    long bh;
    int j0;
    unit_tile<SJ>(p, unit, bh, j0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    const long Tp = static_cast<long>(p.nc) * BC;
    const long SZ = static_cast<long>(DK) * p.dv;
    const long RF = rec_floats<DK>(p.dv);
    f32x4 dacc[NSB];
    load_state_tile<NSB, ST>(p.dST, bh * SZ + j0, p.dv, w, dacc);
#pragma unroll
    for (int m = 0; m < NSB; ++m) {
        const int q = w * NSB + m, ib = ST::sib(q), cb = ST::scb(q);
#pragma unroll
        for (int e = 0; e < 4; ++e) sdS[16 * ib + 4 * g4 + e][16 * cb + ln] = dacc[m][e];
    }
    // X / Y tile of this wave (SJ = 16: waves 2 and 3 compute the tiles of
    // waves 0 and 1 again, which keeps their loads and MFMAs on the same path,
    // and store nothing)
    const int rb = ST::rb(w), xcb = ST::xcb(w);
    const bool xown = w < ST::NXT;
    Tile4<DK, BC * DK / 4> nKg, nQg, nKd;
    Tile4<DK, DK / 4> nGc;
    f32x4 ndO;  // one 4-column group of the dO tile per thread
    float nPt[BC / 4], nMt[BC / 4];  // this lane's P^T and M^T operands: P[4 k + g4][16 rb + ln]
    // dO staging: row dr, columns 4 dc4 .. + 3 (SJ = 16: the upper half of the
    // workgroup loads the rows of the lower half again, stores nothing)
    const int dr = (tid / (SJ / 4)) % BC, dc4 = tid % (SJ / 4);
    auto fetch = [&](long c) {
        const float* R = p.rec + (bh * p.nc + c) * RF;
        nKg.load(R, DK);
        nQg.load(R + BC * DK, DK);
        nKd.load(R + 2 * BC * DK, DK);
        nGc.load(R + rec_gc<DK>(p.dv), DK);
        const float* Rm = R + rec_m<DK>(p.dv);
        const float* Rp = R + rec_p<DK>(p.dv);
#pragma unroll
        for (int k = 0; k < BC / 4; ++k) {
            nPt[k] = Rp[(4 * k + g4) * BC + 16 * rb + ln];
            nMt[k] = Rm[(4 * k + g4) * BC + 16 * rb + ln];
        }
        // clamped row, zeroed past T when staged: a select on the loaded value
        // here would make the compiler wait for every load of the fetch
        ndO = *reinterpret_cast<const f32x4*>(p.dO + (bh * p.T + tclamp(p, c * BC + dr)) * p.dv + j0 + 4 * dc4);
    };
    fetch(p.nc - 1);
    for (long c = p.nc - 1; c >= 0; --c) {
        // gradient with respect to the state after chunk c
#pragma unroll
        for (int m = 0; m < NSB; ++m) {
            const int q = w * NSB + m, ib = ST::sib(q), cb = ST::scb(q);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.dst[(bh * p.nc + c) * SZ + (16 * ib + 4 * g4 + e) * p.dv + j0 + 16 * cb + ln] = dacc[m][e];
        }
        __syncthreads();
        nKg.template store<DK + 4>(&sKg[0][0]);
        nQg.template store<DK + 4>(&sQg[0][0]);
        nKd.template store<DK + 4>(&sKd[0][0]);
        nGc.template store<DK>(sGc);
        if (tid < BC * SJ / 4)
            *reinterpret_cast<f32x4*>(&sdO[dr][4 * dc4]) = c * BC + dr < p.T ? ndO : f32x4{0.f, 0.f, 0.f, 0.f};
        float aPt[BC / 4], aMt[BC / 4];
#pragma unroll
        for (int k = 0; k < BC / 4; ++k) {
            aPt[k] = nPt[k];
            aMt[k] = nMt[k];
        }
        __syncthreads();
        fetch(c > 0 ? c - 1 : 0);  // unconditional, as in the forward pass
        // Y = P^T dO + Kd dS'
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < BC / 4; ++k) y = mfma4(aPt[k], sdO[4 * k + g4][16 * xcb + ln], y);
#pragma unroll
        for (int k = 0; k < DK; k += 4) y = mfma4(sKd[16 * rb + ln][k + g4], sdS[k + g4][16 * xcb + ln], y);
        interleave_loads<BC / 4 + DK / 4>();
        if (xown)
#pragma unroll
            for (int e = 0; e < 4; ++e) sY[16 * rb + 4 * g4 + e][16 * xcb + ln] = y[e];
        __syncthreads();
        // Z = M^T Y, into Y's buffer once every wave has read Y
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < BC / 4; ++k) z = mfma4(aMt[k], sY[4 * k + g4][16 * xcb + ln], z);
        __syncthreads();
        if (xown)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e;
                sY[r][16 * xcb + ln] = z[e];
                p.Z[(bh * Tp + c * BC + r) * p.dv + j0 + 16 * xcb + ln] = z[e];
            }
        __syncthreads();
        // dS <- Diag(e^G_C) dS' + Qg^T dO - Kg^T Z
#pragma unroll
        for (int m = 0; m < NSB; ++m) {
            const int q = w * NSB + m, ib = ST::sib(q), cb = ST::scb(q);
#pragma unroll
            for (int e = 0; e < 4; ++e) dacc[m][e] *= sGc[16 * ib + 4 * g4 + e];
#pragma unroll
            for (int k = 0; k < BC; k += 4) {
                dacc[m] = mfma4(sQg[k + g4][16 * ib + ln], sdO[k + g4][16 * cb + ln], dacc[m]);
                dacc[m] = mfma4(-sKg[k + g4][16 * ib + ln], sY[k + g4][16 * cb + ln], dacc[m]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sdS[16 * ib + 4 * g4 + e][16 * cb + ln] = dacc[m][e];
        }
    }
    if (p.dS0) {
#pragma unroll
        for (int m = 0; m < NSB; ++m) {
            const int q = w * NSB + m, ib = ST::sib(q), cb = ST::scb(q);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.dS0[bh * SZ + (16 * ib + 4 * g4 + e) * p.dv + j0 + 16 * cb + ln] = dacc[m][e];
        }
    }
}

// Both state passes in one launch: the reverse pass needs only the record
// and dO, not the forward states, so the two chains run side by side, one
// workgroup of each per CU, each filling the other's barrier and memory
// waits.  Workgroups are dealt to the XCDs in turn, so the roles alternate
// every kXcds workgroups (every XCD gets both); the grid is padded to
// 2 kXcds per kXcds units and the padding exits at once.
template <int DK, int SJ>
__global__ void __launch_bounds__(NT, 2) bwd_states_kernel(BwdParams p, long units) {
    constexpr int LDSF = fwd_lds_floats<DK, SJ>() > bwd_lds_floats<DK, SJ>() ? fwd_lds_floats<DK, SJ>()
                                                                             : bwd_lds_floats<DK, SJ>();
    __shared__ __attribute__((aligned(16))) float smem[LDSF];
    const long unit = (blockIdx.x / (2 * kXcds)) * kXcds + blockIdx.x % kXcds;
    if (unit >= units) return;  // whole workgroup, before any barrier
    if ((blockIdx.x / kXcds) & 1) state_bwd_body<DK, SJ>(p, smem, unit);
    else state_fwd_body<DK, SJ>(p, smem, unit);
}

// ---------------------------------------------------------------------------
// the dv contractions of one chunk
// ---------------------------------------------------------------------------
// LDS of the dv contractions, in floats
template <int DK>
constexpr int dgrad_lds_floats() { return 2 * DK * (JT + 4) + 3 * BC * (JT + 4); }
// operand buffer of the gate gradients, in floats; dP and dT follow it
template <int DK>
constexpr int gates_sbuf_floats() {
    return 3 * BC * (DK + 16) > 4 * BC * (DK + 1) ? 3 * BC * (DK + 16) : 4 * BC * (DK + 1);
}

// the dv contractions of chunk `unit` (= bh * nc + c): dQg, dKg, dKd and dGamma_C
// into the gradient record, dP and dT into the LDS of the gate phase
template <int DK>
__device__ __forceinline__ void dgrad_body(const BwdParams& p, float* smem, long unit) {
    static_assert(dgrad_lds_floats<DK>() <= gates_sbuf_floats<DK>(),
                  "dP and dT are written above the buffers of this phase");
    constexpr int IBW = DK / 16 / 4;  // 16-channel blocks per wave
    // all read as [row][k]
    float(*sS)[JT + 4] = reinterpret_cast<float(*)[JT + 4]>(smem);
    float(*sE)[JT + 4] = reinterpret_cast<float(*)[JT + 4]>(smem + DK * (JT + 4));
    float(*sdO)[JT + 4] = reinterpret_cast<float(*)[JT + 4]>(smem + 2 * DK * (JT + 4));
    float(*sZ)[JT + 4] = reinterpret_cast<float(*)[JT + 4]>(smem + 2 * DK * (JT + 4) + BC * (JT + 4));
    float(*sU)[JT + 4] = reinterpret_cast<float(*)[JT + 4]>(smem + 2 * DK * (JT + 4) + 2 * BC * (JT + 4));
    const long bh = unit / p.nc;
    const long c = unit % p.nc;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    const long Tp = static_cast<long>(p.nc) * BC;
    const long SZ = static_cast<long>(DK) * p.dv;
    const float* S = p.st + (bh * (p.nc + 1) + c) * SZ;
    const float* E = p.dst + (bh * p.nc + c) * SZ;
    const float* Zc = p.Z + (bh * Tp + c * BC) * p.dv;
    const float* Uc = p.U + (bh * Tp + c * BC) * p.dv;
    f32x4 aQ[2][IBW], aK[2][IBW], aD[2][IBW], aP, aT;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) {
            aQ[rb][ib] = f32x4{0.f, 0.f, 0.f, 0.f};
            aK[rb][ib] = f32x4{0.f, 0.f, 0.f, 0.f};
            aD[rb][ib] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    aP = f32x4{0.f, 0.f, 0.f, 0.f};
    aT = f32x4{0.f, 0.f, 0.f, 0.f};
    const int prb = w >> 1, pcb = w & 1;
    float gacc = 0.f;
    // the next 32 value columns, loaded while the current ones are used
    Tile4<JT, DK * JT / 4> nS, nE;
    Tile4<JT, BC * JT / 4> nZ, nU;
    f32x4 ndO;
    const int dr = tid / (JT / 4), dc4 = tid % (JT / 4);
    auto fetch = [&](int jc) {
        nS.load(S + jc, p.dv);
        nE.load(E + jc, p.dv);
        nZ.load(Zc + jc, p.dv);
        nU.load(Uc + jc, p.dv);
        // clamped row, zeroed past T when staged (see the reverse state pass)
        ndO = *reinterpret_cast<const f32x4*>(p.dO + (bh * p.T + tclamp(p, c * BC + dr)) * p.dv + jc + 4 * dc4);
    };
    const bool dO_row = c * BC + dr < p.T;
    fetch(0);
    for (int jc = 0; jc < p.dv; jc += JT) {
        __syncthreads();
        nS.template store<JT + 4>(&sS[0][0]);
        nE.template store<JT + 4>(&sE[0][0]);
        nZ.template store<JT + 4>(&sZ[0][0]);
        nU.template store<JT + 4>(&sU[0][0]);
        *reinterpret_cast<f32x4*>(&sdO[dr][4 * dc4]) = dO_row ? ndO : f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
        if (jc + JT < p.dv) fetch(jc + JT);
        if (tid < DK)
#pragma unroll 8
            for (int j = 0; j < JT; ++j) gacc += sS[tid][j] * sE[tid][j];
#pragma unroll
        for (int k = 0; k < JT; k += 4) {
            float adO[2], aZ[2], aU[2], bS[IBW], bE[IBW];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                adO[rb] = sdO[16 * rb + ln][k + g4];
                aZ[rb] = sZ[16 * rb + ln][k + g4];
                aU[rb] = sU[16 * rb + ln][k + g4];
            }
#pragma unroll
            for (int ib = 0; ib < IBW; ++ib) {
                bS[ib] = sS[16 * (w * IBW + ib) + ln][k + g4];
                bE[ib] = sE[16 * (w * IBW + ib) + ln][k + g4];
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int ib = 0; ib < IBW; ++ib) {
                    aQ[rb][ib] = mfma4(adO[rb], bS[ib], aQ[rb][ib]);
                    aK[rb][ib] = mfma4(-aZ[rb], bS[ib], aK[rb][ib]);
                    aD[rb][ib] = mfma4(aU[rb], bE[ib], aD[rb][ib]);
                }
            const float bU = sU[16 * pcb + ln][k + g4];
            aP = mfma4(adO[prb], bU, aP);
            aT = mfma4(-aZ[prb], bU, aT);
        }
    }
    float* D = p.dgr + (bh * p.nc + c) * dgr_floats<DK>();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ib = 0; ib < IBW; ++ib)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * g4 + e, i = 16 * (w * IBW + ib) + ln;
                D[r * DK + i] = aQ[rb][ib][e];
                D[BC * DK + r * DK + i] = aK[rb][ib][e];
                D[2 * BC * DK + r * DK + i] = aD[rb][ib][e];
            }
    float(*gdT)[BC + 1] = reinterpret_cast<float(*)[BC + 1]>(smem + gates_sbuf_floats<DK>());
    float(*gdP)[BC + 1] = gdT + BC;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 16 * prb + 4 * g4 + e, s = 16 * pcb + ln;
        gdP[r][s] = s <= r ? aP[e] : 0.f;
        gdT[r][s] = s < r ? aT[e] : 0.f;
    }
    if (tid < DK) D[3 * BC * DK + tid] = gacc;
}

// ---------------------------------------------------------------------------
// from the operand gradients to q, k, v and the gates
//
// The pairwise sums (per key channel i, e_rs = e^(G_ri - G_si) <= 1 for s <= r)
//   A1_r = sum_{s<r} dT_rs kw_s e_rs     A3_r = sum_{s<=r} dP_rs kw_s e_rs
//   A2_s = sum_{r>s} dT_rs kr_r e_rs     A4_s = sum_{r>=s} dP_rs q_r e_rs
// are fp32 MFMA products once e_rs is split at a reference row: inside a
// 16-token block b at its middle row m_b (8 or 24), e_rs = L_r R_s with
// L_r = e^(G_r - G_mb), R_s = e^(G_mb - G_s), both within e^(+-80) by the
// clamp on log alpha; across the blocks (r >= 16 > s) at row 15, where both
// factors are <= 1 and differ from the in-block ones by the per-channel
// constant e^(G_24 - G_8) <= 1.  So with W = kw (.) R, Rk = kr (.) L, Rq = q (.) L:
//   A1 = L (.) [dT W]_in-block + L (.) c (.) [dT_(1,0) W_0]
//   A2 = R (.) [dT^T Rk]_in-block + R (.) c (.) [dT_(1,0)^T Rk_1]   (c = e^(G_24 - G_8))
// and likewise A3, A4 with dP.
// ---------------------------------------------------------------------------

// LDS of the gate gradients, in floats
template <int DK>
constexpr int gates_lds_floats() {
    return gates_sbuf_floats<DK>() + 2 * BC * (BC + 1) + (NT / DK) * 4 * DK + 3 * DK + 3 * BC;
}

// An empty asm statement that may change x, y, z: values derived from them
// past this point are computed afresh rather than reused from earlier
// (register pressure: reuse would keep them live and spill them).
__device__ __forceinline__ void rematerialize(float& x, float& y, float& z) {
    asm volatile("" : "+v"(x), "+v"(y), "+v"(z));
}

// the gate gradients of chunk `unit` (= bh * nc + c), from its gradient record
template <int DK, bool BF16>
__device__ __forceinline__ void gates_body(const BwdParams& p, float* smem, long unit) {
    constexpr int CTW = DK / 16 / 4;  // 16-channel column tiles per wave
    constexpr int OS = DK + 16;       // operand row stride (read as [k][col])
    constexpr int AS = DK + 1;        // result row stride (read per channel)
    constexpr int NH = NT / DK;       // threads per channel
    constexpr int RPT = BC / NH;      // rows per thread
    constexpr int SBUF = gates_sbuf_floats<DK>();
    float* sbuf = smem;  // operands, then A1..A4
    float(*sdT)[BC + 1] = reinterpret_cast<float(*)[BC + 1]>(smem + SBUF);
    float(*sdP)[BC + 1] = reinterpret_cast<float(*)[BC + 1]>(smem + SBUF + BC * (BC + 1));
    // per-part partial sums exchanged between the parts of a channel
    float(*sX)[4][DK] = reinterpret_cast<float(*)[4][DK]>(smem + SBUF + 2 * BC * (BC + 1));
    float(*sRef)[DK] = reinterpret_cast<float(*)[DK]>(smem + SBUF + 2 * BC * (BC + 1) + NH * 4 * DK);  // G_8, G_24, G_C
    float* sRowG = smem + SBUF + 2 * BC * (BC + 1) + NH * 4 * DK + 3 * DK;  // row sums of dgamma'
    float* sMu = sRowG + BC;   // stabilised mode: channel mean of ln(A + eps) per row
    float* sDrm = sMu + BC;    // stabilised mode: channel mean of dr per row
    float(*sW)[OS] = reinterpret_cast<float(*)[OS]>(sbuf);
    float(*sRk)[OS] = reinterpret_cast<float(*)[OS]>(sbuf + BC * OS);
    float(*sRq)[OS] = reinterpret_cast<float(*)[OS]>(sbuf + 2 * BC * OS);
    // A1..A4, then per row: dkr (in A1), dkw (in A3), dG (in A2), dq (in A4);
    // later the per-row sums for scalar gates: d log alpha (A4), dbeta (A1), dA (A3)
    float(*sA1)[AS] = reinterpret_cast<float(*)[AS]>(sbuf);
    float(*sA3)[AS] = reinterpret_cast<float(*)[AS]>(sbuf + BC * AS);
    float(*sA2)[AS] = reinterpret_cast<float(*)[AS]>(sbuf + 2 * BC * AS);
    float(*sA4)[AS] = reinterpret_cast<float(*)[AS]>(sbuf + 3 * BC * AS);
    const long bh = unit / p.nc;
    const long c = unit % p.nc;
    const long t0 = c * BC;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    const long Tp = static_cast<long>(p.nc) * BC;
    const float* D = p.dgr + (bh * p.nc + c) * dgr_floats<DK>();
    if (p.pre && p.stab && tid < BC) sMu[tid] = p.mu[bh * Tp + t0 + tid];
    // thread (channel i, part h) owns rows h RPT .. h RPT + RPT - 1 of channel i;
    // its column is requested first, so these loads overlap those of dv below
    const int i = tid % DK, h = tid / DK, r0 = h * RPT;
    const ColView<DK, BF16> cv(p, bh, t0, i);
    const bool has_decay = p.amode != PDN_ALPHA_NONE;
    float G[RPT], kk[RPT], qv[RPT], bb[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        kk[u] = cv.kv(r0 + u);
        qv[u] = cv.qv(r0 + u);
        G[u] = cv.lav(r0 + u);
        bb[u] = cv.bev(r0 + u);
    }
    // dv and dgamma' (wave w: rows w, w + 4, ...; lanes over columns), in two
    // batches of four rows, every load of a batch before its stores
    const bool gsum = p.gmode == PDN_GATE_SCALAR ||
                      (p.gmode == PDN_GAMMA_SAME_AS_BETA && p.bmode == PDN_GATE_SCALAR);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        float zv[4][4], gv[4][4], vv[4][4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = w + 4 * (4 * half + m);
            const long t = t0 + r;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = min(lane + 64 * u, p.dv - 1);
                zv[m][u] = p.Z[(bh * Tp + t) * p.dv + j];
                gv[m][u] = tok_gamma<DK>(p, bh, t, j);
                vv[m][u] = tok_in<BF16>(p, p.v, bh, t, p.dv, j);
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = w + 4 * (4 * half + m);
            const long t = t0 + r;
            float part = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = lane + 64 * u;
                if (j < p.dv) {
                    const float dg = zv[m][u] * vv[m][u] * value_dscale(p.kmode, p.gmode, gv[m][u]);
                    if (t < p.T) {
                        p.dvo[(bh * p.T + t) * p.dv + j] =
                            zv[m][u] * value_scale(p.kmode, p.gmode, gv[m][u]);
                        if (p.gmode == PDN_GATE_VEC) p.dgamma[(bh * p.T + t) * p.dv + j] = dg;
                    }
                    part += dg;
                }
            }
            if (gsum) {
                part = wave_sum(part);
                if (lane == 0) sRowG[r] = part;
            }
        }
    }
    uint32_t dead = 0;  // own rows whose d log alpha is zero
    float Gin = 0.f, Ain = 0.f;  // cumulative log decay and k (.) k before the own rows
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const bool valid = t0 + r0 + u < p.T;
        if (!valid || !has_decay || G[u] < kLogAlphaMin) dead |= 1u << u;
        G[u] = (valid && has_decay) ? fmaxf(G[u], kLogAlphaMin) : 0.f;
        if (!valid) {
            kk[u] = 0.f;
            qv[u] = 0.f;
            bb[u] = 1.f;
        }
    }
    {
        // prefix over the parts: local sums, exchanged, then made inclusive
        float gs = 0.f, as = 0.f;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            gs += G[u];
            as += kk[u] * kk[u];
        }
        sX[h][0][i] = gs;
        sX[h][1][i] = as;
        __syncthreads();
        for (int h2 = 0; h2 < h; ++h2) {
            Gin += sX[h2][0][i];
            Ain += sX[h2][1][i];
        }
        if (p.pre) Ain += p.apre[(bh * p.nc + c) * DK + i];
        float g = Gin;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            g += G[u];
            G[u] = g;
        }
        // the reference rows 8 and 24 and the last row, for every part of the channel
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int r = r0 + u;
            if (r == 8) sRef[0][i] = G[u];
            if (r == 24) sRef[1][i] = G[u];
            if (r == BC - 1) sRef[2][i] = G[u];
        }
        __syncthreads();
    }
    const float G8 = sRef[0][i], G24 = sRef[1][i], Gc = sRef[2][i];
    // erase gain with the preconditioner folded in, advancing the running sum;
    // aux is the coefficient (1 / (A + eps), or x^-(r / (1 + |r|)) in the
    // stabilised mode, where den = 1 + |r|)
    auto gain_at = [&](int u, float& A, float& aux, float& den) {
        float b = bb[u];
        aux = 1.f;
        den = 1.f;
        if (p.pre) {
            A += kk[u] * kk[u];
            if (p.stab) {
                const float x = logf(A + p.eps) - sMu[r0 + u];
                den = 1.f + fabsf(x);
                aux = __expf(-(x / den) * p.lnx);
            } else {
                aux = 1.f / (A + p.eps);
            }
            b = b * aux;
        }
        return b;
    };
    {
        float A = Ain, aux, den;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int r = r0 + u;
            float kwr, krr;
            keys_of(p.kmode, gain_at(u, A, aux, den), kk[u], kwr, krr);
            const float gm = r < 16 ? G8 : G24;
            const float L = __expf(G[u] - gm), R = __expf(gm - G[u]);
            sW[r][i] = kwr * R;
            sRk[r][i] = krr * L;
            sRq[r][i] = qv[u] * L;
        }
    }
    __syncthreads();
    // MFMA: wave w, column tiles CTW w .. CTW w + CTW - 1
    f32x4 a1[CTW][2], a3[CTW][2], a2[CTW][2], a4[CTW][2];
#pragma unroll
    for (int m = 0; m < CTW; ++m) {
        const int col = 16 * (CTW * w + m) + ln;
        f32x4 x1[3], x3[3], x2[3], x4[3];  // [in block 0, in block 1, across]
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            x1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            x3[u] = x1[u];
            x2[u] = x1[u];
            x4[u] = x1[u];
        }
#pragma unroll
        for (int k = 0; k < 16; k += 4) {
            const int kk0 = k + g4, kk1 = 16 + k + g4;
            const float w0 = sW[kk0][col], w1 = sW[kk1][col];
            const float rk0 = sRk[kk0][col], rk1 = sRk[kk1][col];
            const float rq0 = sRq[kk0][col], rq1 = sRq[kk1][col];
            // r side: rows of block b times the W rows of the s block
            x1[0] = mfma4(sdT[ln][kk0], w0, x1[0]);
            x1[1] = mfma4(sdT[16 + ln][kk1], w1, x1[1]);
            x1[2] = mfma4(sdT[16 + ln][kk0], w0, x1[2]);
            x3[0] = mfma4(sdP[ln][kk0], w0, x3[0]);
            x3[1] = mfma4(sdP[16 + ln][kk1], w1, x3[1]);
            x3[2] = mfma4(sdP[16 + ln][kk0], w0, x3[2]);
            // s side: transposed blocks times the Rk / Rq rows of the r block
            x2[0] = mfma4(sdT[kk0][ln], rk0, x2[0]);
            x2[1] = mfma4(sdT[kk1][16 + ln], rk1, x2[1]);
            x2[2] = mfma4(sdT[kk1][ln], rk1, x2[2]);
            x4[0] = mfma4(sdP[kk0][ln], rq0, x4[0]);
            x4[1] = mfma4(sdP[kk1][16 + ln], rq1, x4[1]);
            x4[2] = mfma4(sdP[kk1][ln], rq1, x4[2]);
        }
        const float cst = __expf(sRef[1][col] - sRef[0][col]);  // e^(G_24 - G_8)
        a1[m][0] = x1[0];
        a3[m][0] = x3[0];
        a2[m][1] = x2[1];
        a4[m][1] = x4[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a1[m][1][e] = x1[1][e] + cst * x1[2][e];
            a3[m][1][e] = x3[1][e] + cst * x3[2][e];
            a2[m][0][e] = x2[0][e] + cst * x2[2][e];
            a4[m][0][e] = x4[0][e] + cst * x4[2][e];
        }
    }
    __syncthreads();  // every wave has read the operands: the buffer takes A1..A4
#pragma unroll
    for (int m = 0; m < CTW; ++m) {
        const int col = 16 * (CTW * w + m) + ln;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * b + 4 * g4 + e;
                sA1[r][col] = a1[m][b][e];
                sA3[r][col] = a3[m][b][e];
                sA2[r][col] = a2[m][b][e];
                sA4[r][col] = a4[m][b][e];
            }
    }
    __syncthreads();
    const float* DdQg = D + i;
    const float* DdKg = D + BC * DK + i;
    const float* DdKd = D + 2 * BC * DK + i;
    // dGamma_C of channel i, read with the rows below: read at the start of the
    // phase, the compiler spilled it at once, and the spill store waited for
    // every load issued before it (the channel columns)
    const float dgam = D[3 * BC * DK + i];
    float kdsum = 0.f;
    {
        float dqg[RPT], dkg[RPT], dkd[RPT];
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            dqg[u] = DdQg[(r0 + u) * DK];
            dkg[u] = DdKg[(r0 + u) * DK];
            dkd[u] = DdKd[(r0 + u) * DK];
        }
        float A = Ain, aux, den;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int r = r0 + u;
            // the gains and decay factors of the operand step are recomputed
            // here, not kept: left to itself the compiler reuses them, keeps
            // 16 rows of them live across the MFMA step, spills them, and
            // reloads one per row, each reload waiting for every load in flight
            rematerialize(G[u], kk[u], bb[u]);
            float kwr, krr;
            keys_of(p.kmode, gain_at(u, A, aux, den), kk[u], kwr, krr);
            const float gm = r < 16 ? G8 : G24;
            const float L = __expf(G[u] - gm), R = __expf(gm - G[u]);
            const float A1 = L * sA1[r][i], A3 = L * sA3[r][i];
            const float A2 = R * sA2[r][i], A4 = R * sA4[r][i];
            const float eg = __expf(G[u]);
            const float ed = __expf(Gc - G[u]);
            const float kd = kwr * ed;
            kdsum += dkd[u] * kd;
            sA4[r][i] = dqg[u] * eg + A3;         // dq
            sA1[r][i] = dkg[u] * eg + A1;         // dkr
            sA3[r][i] = dkd[u] * ed + A2 + A4;    // dkw
            sA2[r][i] = dkg[u] * krr * eg + dqg[u] * qv[u] * eg + krr * A1 + qv[u] * A3 -
                        dkd[u] * kd - kwr * (A2 + A4);  // dG
        }
    }
    sX[h][2][i] = kdsum;
    __syncthreads();
    if (h == NH - 1) {
        float tot = 0.f;
#pragma unroll
        for (int h2 = 0; h2 < NH; ++h2) tot += sX[h2][2][i];
        sA2[BC - 1][i] += tot + dgam * __expf(Gc);
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u)
        if (t0 + r0 + u < p.T) p.dq[(bh * p.T + t0 + r0 + u) * DK + i] = sA4[r0 + u][i];
    // dG totals of the parts, for the reverse cumulative sum across them
    {
        float tot = 0.f;
#pragma unroll
        for (int u = 0; u < RPT; ++u) tot += sA2[r0 + u][i];
        sX[h][3][i] = tot;
    }
    __syncthreads();
    {
        // d log alpha: reverse cumulative sum of dG over the chunk
        float run = 0.f;
        for (int h2 = h + 1; h2 < NH; ++h2) run += sX[h2][3][i];
#pragma unroll
        for (int u = RPT - 1; u >= 0; --u) {
            const int r = r0 + u;
            run += sA2[r][i];
            sA4[r][i] = ((dead >> u) & 1u) ? 0.f : run;
        }
        // stored after the loop: a store between the steps above would make
        // each step's register reload wait for it (one counter serves both)
        if (p.amode == PDN_ALPHA_VEC)
#pragma unroll
            for (int u = 0; u < RPT; ++u)
                if (t0 + r0 + u < p.T) p.dla[(bh * p.T + t0 + r0 + u) * DK + i] = sA4[r0 + u][i];
        // keys to k and the gains; the preconditioner's dA (the stabilised mode
        // first leaves dr in A2 for its channel mean)
        float A = Ain, aux, den;
        float dAsum = 0.f;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int r = r0 + u;
            const long t = t0 + r;
            rematerialize(G[u], kk[u], bb[u]);  // as in the per-row step above
            const float braw = bb[u];
            const float b = gain_at(u, A, aux, den);
            const float dkwr = sA3[r][i], dkrr = sA1[r][i];
            float dkk, db;
            if (p.kmode == PDN_KEY_SYMMETRIC) {
                const float sb = sqrtf(b);
                dkk = (dkwr + dkrr) * sb;
                db = (dkwr + dkrr) * kk[u] * 0.5f / sb;
            } else if (p.kmode == PDN_KEY_ERASE_GATE) {
                dkk = dkwr + dkrr * b;
                db = dkrr * kk[u];
            } else {
                dkk = dkwr * b + dkrr;
                db = dkwr * kk[u];
            }
            float dA = 0.f;
            if (p.pre) {
                if (p.stab) {
                    // B = x^-s, s = x_r / (1 + |x_r|), x_r = ln(A + eps) - mean
                    sA2[r][i] = -db * braw * aux * p.lnx / (den * den);
                } else {
                    dA = -db * braw * aux * aux;
                }
                db *= aux;
            }
            if (p.gmode == PDN_GAMMA_SAME_AS_BETA && p.bmode == PDN_GATE_VEC && t < p.T) {
                // beta also scales the value of column i (dk == dv)
                const float z = p.Z[(bh * Tp + t) * p.dv + i];
                const float vv = load_in<BF16>(p.v, (bh * p.T + t) * p.dv + i);
                db += z * vv * value_dscale(p.kmode, p.gmode, braw);
            }
            if (t < p.T) {
                p.dk[(bh * p.T + t) * DK + i] = dkk;
                if (p.bmode == PDN_GATE_VEC) p.dbeta[(bh * p.T + t) * DK + i] = db;
            }
            sA1[r][i] = db;
            sA3[r][i] = dA;
            dAsum += dA;
        }
        if (p.pre) sX[h][0][i] = dAsum;
    }
    __syncthreads();
    if (p.pre && p.stab) {
        // dl = dr - mean over channels of dr; dA = dl / (A + eps)
        if (tid < BC) {
            float m = 0.f;
            for (int ii = 0; ii < DK; ++ii) m += sA2[tid][ii];
            sDrm[tid] = m * (1.f / DK);
        }
        __syncthreads();
        float A = Ain, dAsum = 0.f;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int r = r0 + u;
            A += kk[u] * kk[u];
            const float dA = (sA2[r][i] - sDrm[r]) / (A + p.eps);
            sA3[r][i] = dA;
            dAsum += dA;
        }
        sX[h][0][i] = dAsum;
        __syncthreads();
    }
    if (p.pre) {
        float suf = 0.f;
        for (int h2 = h + 1; h2 < NH; ++h2) suf += sX[h2][0][i];
#pragma unroll
        for (int u = RPT - 1; u >= 0; --u) {
            suf += sA3[r0 + u][i];
            p.dAin[(bh * Tp + t0 + r0 + u) * DK + i] = suf;
        }
        if (h == 0) p.dAc[(bh * p.nc + c) * DK + i] = suf;
    }
    // per-token sums for scalar gates
    if (tid < BC) {
        const int r = tid;
        const long t = t0 + r;
        if (t < p.T) {
            if (p.amode == PDN_ALPHA_SCALAR) {
                float sm = 0.f;
                for (int ii = 0; ii < DK; ++ii) sm += sA4[r][ii];
                p.dla[bh * p.T + t] = sm;
            }
            if (p.bmode == PDN_GATE_SCALAR) {
                float sm = 0.f;
                for (int ii = 0; ii < DK; ++ii) sm += sA1[r][ii];
                if (p.gmode == PDN_GAMMA_SAME_AS_BETA) sm += sRowG[r];
                p.dbeta[bh * p.T + t] = sm;
            }
            if (p.gmode == PDN_GATE_SCALAR) p.dgamma[bh * p.T + t] = sRowG[r];
        }
    }
}

// The dv contractions and the gate gradients of one chunk in one workgroup:
// the gradient record goes out and comes back through L2, and two
// workgroups per CU overlap one's MFMA-heavy contractions with the other's
// gate work.
template <int DK, bool BF16>
__global__ void __launch_bounds__(NT, 2) bwd_grads_kernel(BwdParams p) {
    constexpr int LDSF = dgrad_lds_floats<DK>() > gates_lds_floats<DK>() ? dgrad_lds_floats<DK>()
                                                                         : gates_lds_floats<DK>();
    __shared__ __attribute__((aligned(16))) float smem[LDSF];
    dgrad_body<DK>(p, smem, blockIdx.x);
    __syncthreads();  // the record written by every thread is visible to the workgroup
    gates_body<DK, BF16>(p, smem, blockIdx.x);
}

// ---------------------------------------------------------------------------
// preconditioner: dk += 2 k (.) sum_{s >= t} dA_s, dA0
// ---------------------------------------------------------------------------

template <int DK, bool BF16>
__global__ void __launch_bounds__(NT) bwd_dA_apply_kernel(BwdParams p) {
    const long bh = blockIdx.x / p.nc;
    const long c = blockIdx.x % p.nc;
    const long Tp = static_cast<long>(p.nc) * BC;
    for (int idx = threadIdx.x; idx < BC * DK; idx += NT) {
        const int r = idx / DK, i = idx % DK;
        const long t = c * BC + r;
        if (t >= p.T) continue;
        const float kk = load_in<BF16>(p.k, (bh * p.T + t) * DK + i);
        p.dk[(bh * p.T + t) * DK + i] +=
            2.f * kk * (p.dAin[(bh * Tp + t) * DK + i] + p.dAsuf[(bh * p.nc + c) * DK + i]);
    }
}

}  // namespace
}  // namespace pdn
