// Backward of the chunked gated delta rule on gfx950: gradients of
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
//   bwd_ksum / bwd_kscan   preconditioner: running k (.) k before each chunk
//   bwd_prep               per chunk: Kg, Qg, Kd, Vw, M, P, e^G_C (the record)
//   bwd_state_fwd          per (b, h, 32 value columns), chunks in order: the
//                          chunk start states S and U
//   bwd_state_bwd          same, chunks in reverse: dS' per chunk, Z, dS0
//   bwd_dgrad              per chunk: the dv contractions (dQg, dKg, dKd, dP,
//                          dT, dGamma_C), fp32 16x16x4 MFMAs
//   bwd_gates              per chunk and key channel: dq, dk, dv, d log alpha,
//                          dbeta, dgamma, and the preconditioner's dA
//   bwd_dA_scan / bwd_dA_apply   preconditioner: dk += 2 k (.) sum_{s>=t} dA_s
//
// Every product is an fp32 MFMA (exact fp32 products, fp32 accumulation) or
// fp32 VALU; the pairwise decays are exact exponentials, so no clamp-driven
// splitting is needed here (log alpha is still clamped at -10 as in the
// forward, with zero gradient where it clamps).
#include "common.h"
#include "kernels.h"

namespace pdn {
namespace {

constexpr int BC = 32;   // tokens per chunk
constexpr int NT = 256;  // threads per workgroup (four waves)
constexpr int JT = 32;   // value columns per state tile

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

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
};

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
__host__ __device__ constexpr long dgr_floats() { return 3L * BC * DK + 2L * BC * BC + DK; }

// ---------------------------------------------------------------------------
// per-token gates (shared by the prep and the gradient kernels)
// ---------------------------------------------------------------------------

// clamped natural-log decay of token t (0 beyond T or without decay)
template <int DK>
__device__ __forceinline__ float tok_la(const BwdParams& p, long bh, long t, int i) {
    if (t >= p.T || p.amode == PDN_ALPHA_NONE) return 0.f;
    const float x = p.amode == PDN_ALPHA_SCALAR ? p.la[bh * p.T + t] : p.la[(bh * p.T + t) * DK + i];
    return fmaxf(x, kLogAlphaMin);
}
template <int DK>
__device__ __forceinline__ bool tok_la_clamped(const BwdParams& p, long bh, long t, int i) {
    if (t >= p.T || p.amode == PDN_ALPHA_NONE) return true;
    const float x = p.amode == PDN_ALPHA_SCALAR ? p.la[bh * p.T + t] : p.la[(bh * p.T + t) * DK + i];
    return x < kLogAlphaMin;
}
// raw erase gain (1 beyond T, so that padded rows carry finite zero gradients)
template <int DK>
__device__ __forceinline__ float tok_beta(const BwdParams& p, long bh, long t, int i) {
    if (t >= p.T) return 1.f;
    return p.bmode == PDN_GATE_SCALAR ? p.beta[bh * p.T + t] : p.beta[(bh * p.T + t) * DK + i];
}
// raw value gain of column j (raw beta when gamma is "same as beta")
template <int DK>
__device__ __forceinline__ float tok_gamma(const BwdParams& p, long bh, long t, int j) {
    if (t >= p.T) return 1.f;
    if (p.gmode == PDN_GAMMA_SAME_AS_BETA)
        return p.bmode == PDN_GATE_SCALAR ? p.beta[bh * p.T + t] : p.beta[(bh * p.T + t) * DK + j];
    return p.gmode == PDN_GATE_SCALAR ? p.gamma[bh * p.T + t] : p.gamma[(bh * p.T + t) * p.dv + j];
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

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, long i) {
    return load_in<BF16>(p, i);
}

// ---------------------------------------------------------------------------
// preconditioner: A before each chunk
// ---------------------------------------------------------------------------
template <int DK, bool BF16>
__global__ void __launch_bounds__(DK) bwd_ksum_kernel(BwdParams p) {
    const long bh = blockIdx.x / p.nc;
    const long c = blockIdx.x % p.nc;
    const int i = threadIdx.x;
    float s = 0.f;
    for (int r = 0; r < BC; ++r) {
        const long t = c * BC + r;
        if (t < p.T) {
            const float kk = ld<BF16>(p.k, (bh * p.T + t) * DK + i);
            s += kk * kk;
        }
    }
    p.ksum[(bh * p.nc + c) * DK + i] = s;
}

template <int DK>
__global__ void __launch_bounds__(DK) bwd_kscan_kernel(BwdParams p) {
    const long bh = blockIdx.x;
    const int i = threadIdx.x;
    float run = p.A0 ? p.A0[bh * DK + i] : 0.f;
    for (long c = 0; c < p.nc; ++c) {
        p.apre[(bh * p.nc + c) * DK + i] = run;
        run += p.ksum[(bh * p.nc + c) * DK + i];
    }
}

// ---------------------------------------------------------------------------
// per-chunk record
// ---------------------------------------------------------------------------
template <int DK, bool BF16>
__global__ void __launch_bounds__(NT) bwd_prep_kernel(BwdParams p) {
    __shared__ float sKr[BC][DK + 1];
    __shared__ float sKw[BC][DK + 1];
    __shared__ float sQ[BC][DK + 1];
    __shared__ float sG[BC][DK + 1];  // log2 units
    __shared__ float sT[BC][BC + 1];
    __shared__ float sM[BC][BC + 1];
    const long bh = blockIdx.x / p.nc;
    const long c = blockIdx.x % p.nc;
    const long t0 = c * BC;
    const int tid = threadIdx.x;
    float* R = p.rec + (bh * p.nc + c) * rec_floats<DK>(p.dv);
    if (tid < DK) {
        const int i = tid;
        float G = 0.f;
        float A = p.pre ? p.apre[(bh * p.nc + c) * DK + i] : 0.f;
        for (int r = 0; r < BC; ++r) {
            const long t = t0 + r;
            const float kk = t < p.T ? ld<BF16>(p.k, (bh * p.T + t) * DK + i) : 0.f;
            const float qq = t < p.T ? ld<BF16>(p.q, (bh * p.T + t) * DK + i) : 0.f;
            G += tok_la<DK>(p, bh, t, i);
            float b = tok_beta<DK>(p, bh, t, i);
            if (p.pre) {
                A += kk * kk;
                b = b / (A + p.eps);
            }
            float kw, kr;
            keys_of(p.kmode, b, kk, kw, kr);
            sKr[r][i] = kr;
            sKw[r][i] = kw;
            sQ[r][i] = qq;
            sG[r][i] = G * kLog2e;
        }
        const float gc = G * kLog2e;
        for (int r = 0; r < BC; ++r) {
            const float e = exp2f(sG[r][i]);
            R[r * DK + i] = sKr[r][i] * e;
            R[BC * DK + r * DK + i] = sQ[r][i] * e;
            R[2 * BC * DK + r * DK + i] = sKw[r][i] * exp2f(gc - sG[r][i]);
        }
        R[rec_gc<DK>(p.dv) + i] = exp2f(gc);
    }
    float* Rvw = R + rec_vw<DK>(p.dv);
    for (int idx = tid; idx < BC * p.dv; idx += NT) {
        const int r = idx / p.dv, j = idx % p.dv;
        const long t = t0 + r;
        const float vv = t < p.T ? ld<BF16>(p.v, (bh * p.T + t) * p.dv + j) : 0.f;
        Rvw[idx] = vv * value_scale(p.kmode, p.gmode, tok_gamma<DK>(p, bh, t, j));
    }
    __syncthreads();
    float* Rp = R + rec_p<DK>(p.dv);
    for (int idx = tid; idx < BC * BC; idx += NT) {
        const int r = idx / BC, s = idx % BC;
        float tv = 0.f, pv = 0.f;
        if (s <= r) {
            for (int i = 0; i < DK; ++i) {
                const float w = sKw[s][i] * exp2f(sG[r][i] - sG[s][i]);
                tv += sKr[r][i] * w;
                pv += sQ[r][i] * w;
            }
        }
        sT[r][s] = s < r ? tv : 0.f;
        Rp[idx] = pv;  // zero above the diagonal
    }
    __syncthreads();
    // M = (I + T)^-1, one column per thread: x_r = [r == j] - sum_{s<r} T_rs x_s
    if (tid < BC) {
        const int j = tid;
        for (int r = 0; r < BC; ++r) {
            float acc = r == j ? 1.f : 0.f;
            for (int s = j; s < r; ++s) acc -= sT[r][s] * sM[s][j];
            sM[r][j] = r < j ? 0.f : acc;
        }
    }
    __syncthreads();
    float* Rm = R + rec_m<DK>(p.dv);
    for (int idx = tid; idx < BC * BC; idx += NT) Rm[idx] = sM[idx / BC][idx % BC];
}

// ---------------------------------------------------------------------------
// state passes: one workgroup per (b, h, 32 value columns); state tile
// DK x 32 in MFMA accumulators, (DK / 16) x 2 tiles of 16 x 16 over 4 waves.
// ---------------------------------------------------------------------------
template <int DK>
__global__ void __launch_bounds__(NT) bwd_state_fwd_kernel(BwdParams p) {
    constexpr int NSB = DK / 16 * 2 / 4;  // state tiles per wave
    __shared__ float sKg[BC][DK + 4];     // read as [row][k]: stride 4 mod 64 banks
    __shared__ float sKd[BC][DK + 16];    // read as [k][col]: stride 16 mod 64
    __shared__ float sM[BC][BC + 4];
    __shared__ float sX[BC][JT + 16];
    __shared__ float sU[BC][JT + 16];
    __shared__ float sS[DK][JT + 16];
    __shared__ float sGc[DK];
    const int ntile = p.dv / JT;
    const long bh = blockIdx.x / ntile;
    const int j0 = (blockIdx.x % ntile) * JT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    const long Tp = static_cast<long>(p.nc) * BC;
    const long SZ = static_cast<long>(DK) * p.dv;
    f32x4 sacc[NSB];
#pragma unroll
    for (int m = 0; m < NSB; ++m) {
        const int q = w * NSB + m, ib = q >> 1, cb = q & 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * ib + 4 * g4 + e, col = 16 * cb + ln;
            const float v = p.S0 ? p.S0[bh * SZ + row * p.dv + j0 + col] : 0.f;
            sacc[m][e] = v;
            sS[row][col] = v;
            p.st[bh * (p.nc + 1) * SZ + row * p.dv + j0 + col] = v;
        }
    }
    const int rb = w >> 1, xcb = w & 1;
    for (long c = 0; c < p.nc; ++c) {
        const float* R = p.rec + (bh * p.nc + c) * rec_floats<DK>(p.dv);
        __syncthreads();
        for (int idx = tid; idx < BC * DK; idx += NT) {
            const int r = idx / DK, i = idx % DK;
            sKg[r][i] = R[idx];
            sKd[r][i] = R[2 * BC * DK + idx];
        }
        const float* Rm = R + rec_m<DK>(p.dv);
        for (int idx = tid; idx < BC * BC; idx += NT) sM[idx / BC][idx % BC] = Rm[idx];
        for (int i = tid; i < DK; i += NT) sGc[i] = R[rec_gc<DK>(p.dv) + i];
        __syncthreads();
        // X = Vw - Kg S: tile (rb, xcb)
        const float* Rvw = R + rec_vw<DK>(p.dv);
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = Rvw[(16 * rb + 4 * g4 + e) * p.dv + j0 + 16 * xcb + ln];
#pragma unroll 8
        for (int k = 0; k < DK; k += 4) x = mfma4(-sKg[16 * rb + ln][k + g4], sS[k + g4][16 * xcb + ln], x);
#pragma unroll
        for (int e = 0; e < 4; ++e) sX[16 * rb + 4 * g4 + e][16 * xcb + ln] = x[e];
        __syncthreads();
        // U = M X
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < BC; k += 4) u = mfma4(sM[16 * rb + ln][k + g4], sX[k + g4][16 * xcb + ln], u);
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
            const int q = w * NSB + m, ib = q >> 1, cb = q & 1;
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

template <int DK>
__global__ void __launch_bounds__(NT) bwd_state_bwd_kernel(BwdParams p) {
    constexpr int NSB = DK / 16 * 2 / 4;
    __shared__ float sQg[BC][DK + 16];  // read as [k][col]
    __shared__ float sKg[BC][DK + 16];
    __shared__ float sKd[BC][DK + 4];   // read as [row][k]
    __shared__ float sM[BC][BC + 16];   // read transposed: [k][col]
    __shared__ float sP[BC][BC + 16];
    __shared__ float sdO[BC][JT + 16];
    __shared__ float sY[BC][JT + 16];
    __shared__ float sZ[BC][JT + 16];
    __shared__ float sdS[DK][JT + 16];
    __shared__ float sGc[DK];
    const int ntile = p.dv / JT;
    const long bh = blockIdx.x / ntile;
    const int j0 = (blockIdx.x % ntile) * JT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    const long Tp = static_cast<long>(p.nc) * BC;
    const long SZ = static_cast<long>(DK) * p.dv;
    f32x4 dacc[NSB];
#pragma unroll
    for (int m = 0; m < NSB; ++m) {
        const int q = w * NSB + m, ib = q >> 1, cb = q & 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * ib + 4 * g4 + e, col = 16 * cb + ln;
            const float v = p.dST ? p.dST[bh * SZ + row * p.dv + j0 + col] : 0.f;
            dacc[m][e] = v;
            sdS[row][col] = v;
        }
    }
    const int rb = w >> 1, xcb = w & 1;
    for (long c = p.nc - 1; c >= 0; --c) {
        // gradient with respect to the state after chunk c
#pragma unroll
        for (int m = 0; m < NSB; ++m) {
            const int q = w * NSB + m, ib = q >> 1, cb = q & 1;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.dst[(bh * p.nc + c) * SZ + (16 * ib + 4 * g4 + e) * p.dv + j0 + 16 * cb + ln] = dacc[m][e];
        }
        const float* R = p.rec + (bh * p.nc + c) * rec_floats<DK>(p.dv);
        __syncthreads();
        for (int idx = tid; idx < BC * DK; idx += NT) {
            const int r = idx / DK, i = idx % DK;
            sKg[r][i] = R[idx];
            sQg[r][i] = R[BC * DK + idx];
            sKd[r][i] = R[2 * BC * DK + idx];
        }
        const float* Rm = R + rec_m<DK>(p.dv);
        const float* Rp = R + rec_p<DK>(p.dv);
        for (int idx = tid; idx < BC * BC; idx += NT) {
            sM[idx / BC][idx % BC] = Rm[idx];
            sP[idx / BC][idx % BC] = Rp[idx];
        }
        for (int i = tid; i < DK; i += NT) sGc[i] = R[rec_gc<DK>(p.dv) + i];
        for (int idx = tid; idx < BC * JT; idx += NT) {
            const int r = idx / JT, j = idx % JT;
            const long t = c * BC + r;
            sdO[r][j] = t < p.T ? p.dO[(bh * p.T + t) * p.dv + j0 + j] : 0.f;
        }
        __syncthreads();
        // Y = P^T dO + Kd dS'
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < BC; k += 4) y = mfma4(sP[k + g4][16 * rb + ln], sdO[k + g4][16 * xcb + ln], y);
#pragma unroll 8
        for (int k = 0; k < DK; k += 4) y = mfma4(sKd[16 * rb + ln][k + g4], sdS[k + g4][16 * xcb + ln], y);
#pragma unroll
        for (int e = 0; e < 4; ++e) sY[16 * rb + 4 * g4 + e][16 * xcb + ln] = y[e];
        __syncthreads();
        // Z = M^T Y
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < BC; k += 4) z = mfma4(sM[k + g4][16 * rb + ln], sY[k + g4][16 * xcb + ln], z);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e;
            sZ[r][16 * xcb + ln] = z[e];
            p.Z[(bh * Tp + c * BC + r) * p.dv + j0 + 16 * xcb + ln] = z[e];
        }
        __syncthreads();
        // dS <- Diag(e^G_C) dS' + Qg^T dO - Kg^T Z
#pragma unroll
        for (int m = 0; m < NSB; ++m) {
            const int q = w * NSB + m, ib = q >> 1, cb = q & 1;
#pragma unroll
            for (int e = 0; e < 4; ++e) dacc[m][e] *= sGc[16 * ib + 4 * g4 + e];
#pragma unroll
            for (int k = 0; k < BC; k += 4) {
                dacc[m] = mfma4(sQg[k + g4][16 * ib + ln], sdO[k + g4][16 * cb + ln], dacc[m]);
                dacc[m] = mfma4(-sKg[k + g4][16 * ib + ln], sZ[k + g4][16 * cb + ln], dacc[m]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sdS[16 * ib + 4 * g4 + e][16 * cb + ln] = dacc[m][e];
        }
    }
    if (p.dS0) {
#pragma unroll
        for (int m = 0; m < NSB; ++m) {
            const int q = w * NSB + m, ib = q >> 1, cb = q & 1;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.dS0[bh * SZ + (16 * ib + 4 * g4 + e) * p.dv + j0 + 16 * cb + ln] = dacc[m][e];
        }
    }
}

// ---------------------------------------------------------------------------
// the dv contractions of one chunk
// ---------------------------------------------------------------------------
template <int DK>
__global__ void __launch_bounds__(NT) bwd_dgrad_kernel(BwdParams p) {
    constexpr int IBW = DK / 16 / 4;  // 16-channel blocks per wave
    __shared__ float sS[DK][JT + 4];  // all read as [row][k]
    __shared__ float sE[DK][JT + 4];
    __shared__ float sdO[BC][JT + 4];
    __shared__ float sZ[BC][JT + 4];
    __shared__ float sU[BC][JT + 4];
    const long bh = blockIdx.x / p.nc;
    const long c = blockIdx.x % p.nc;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    const long Tp = static_cast<long>(p.nc) * BC;
    const long SZ = static_cast<long>(DK) * p.dv;
    const float* S = p.st + (bh * (p.nc + 1) + c) * SZ;
    const float* E = p.dst + (bh * p.nc + c) * SZ;
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
    for (int jc = 0; jc < p.dv; jc += JT) {
        __syncthreads();
        for (int idx = tid; idx < DK * JT; idx += NT) {
            const int i = idx / JT, j = idx % JT;
            sS[i][j] = S[i * p.dv + jc + j];
            sE[i][j] = E[i * p.dv + jc + j];
        }
        for (int idx = tid; idx < BC * JT; idx += NT) {
            const int r = idx / JT, j = idx % JT;
            const long t = c * BC + r;
            sdO[r][j] = t < p.T ? p.dO[(bh * p.T + t) * p.dv + jc + j] : 0.f;
            sZ[r][j] = p.Z[(bh * Tp + c * BC + r) * p.dv + jc + j];
            sU[r][j] = p.U[(bh * Tp + c * BC + r) * p.dv + jc + j];
        }
        __syncthreads();
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
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 16 * prb + 4 * g4 + e, s = 16 * pcb + ln;
        D[3 * BC * DK + r * BC + s] = s <= r ? aP[e] : 0.f;
        D[3 * BC * DK + BC * BC + r * BC + s] = s < r ? aT[e] : 0.f;
    }
    if (tid < DK) D[3 * BC * DK + 2 * BC * BC + tid] = gacc;
}

// ---------------------------------------------------------------------------
// from the operand gradients to q, k, v and the gates
// ---------------------------------------------------------------------------
template <int DK, bool BF16>
__global__ void __launch_bounds__(NT) bwd_gates_kernel(BwdParams p) {
    __shared__ float sKr[BC][DK + 1];
    __shared__ float sKw[BC][DK + 1];
    __shared__ float sQ[BC][DK + 1];
    __shared__ float sG[BC][DK + 1];  // natural log
    __shared__ float sdT[BC][BC + 1];
    __shared__ float sdP[BC][BC + 1];
    __shared__ float sW[BC][DK + 1];   // dKw, then the per-row dbeta terms
    __shared__ float sDG[BC][DK + 1];  // dG (s side), then d log alpha
    __shared__ float sRowG[BC];        // row sums of dgamma'
    const long bh = blockIdx.x / p.nc;
    const long c = blockIdx.x % p.nc;
    const long t0 = c * BC;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const long Tp = static_cast<long>(p.nc) * BC;
    const float* D = p.dgr + (bh * p.nc + c) * dgr_floats<DK>();
    const float* DdQg = D;
    const float* DdKg = D + BC * DK;
    const float* DdKd = D + 2 * BC * DK;
    const float* DdGc = D + 3 * BC * DK + 2 * BC * BC;
    for (int idx = tid; idx < BC * BC; idx += NT) {
        sdP[idx / BC][idx % BC] = D[3 * BC * DK + idx];
        sdT[idx / BC][idx % BC] = D[3 * BC * DK + BC * BC + idx];
    }
    // dv and dgamma' (wave w: rows w, w + 4, ...)
    const bool gsum = p.gmode == PDN_GATE_SCALAR || (p.gmode == PDN_GAMMA_SAME_AS_BETA && p.bmode == PDN_GATE_SCALAR);
    for (int r = w; r < BC; r += 4) {
        const long t = t0 + r;
        float part = 0.f;
        for (int j = lane; j < p.dv; j += 64) {
            const float z = p.Z[(bh * Tp + t) * p.dv + j];
            const float g = tok_gamma<DK>(p, bh, t, j);
            const float vv = t < p.T ? ld<BF16>(p.v, (bh * p.T + t) * p.dv + j) : 0.f;
            const float dg = z * vv * value_dscale(p.kmode, p.gmode, g);
            if (t < p.T) {
                p.dvo[(bh * p.T + t) * p.dv + j] = z * value_scale(p.kmode, p.gmode, g);
                if (p.gmode == PDN_GATE_VEC) p.dgamma[(bh * p.T + t) * p.dv + j] = dg;
            }
            part += dg;
        }
        if (gsum) {
            part = wave_sum(part);
            if (lane == 0) sRowG[r] = part;
        }
    }
    const int i = tid % DK, part = tid / DK;
    // per-channel columns of the chunk (part 0)
    if (part == 0) {
        float G = 0.f;
        float A = p.pre ? p.apre[(bh * p.nc + c) * DK + i] : 0.f;
        for (int r = 0; r < BC; ++r) {
            const long t = t0 + r;
            const float kk = t < p.T ? ld<BF16>(p.k, (bh * p.T + t) * DK + i) : 0.f;
            const float qq = t < p.T ? ld<BF16>(p.q, (bh * p.T + t) * DK + i) : 0.f;
            G += tok_la<DK>(p, bh, t, i);
            float b = tok_beta<DK>(p, bh, t, i);
            if (p.pre) {
                A += kk * kk;
                b = b / (A + p.eps);
            }
            float kw, kr;
            keys_of(p.kmode, b, kk, kw, kr);
            sKr[r][i] = kr;
            sKw[r][i] = kw;
            sQ[r][i] = qq;
            sG[r][i] = G;
        }
    }
    __syncthreads();
    const float Gc = sG[BC - 1][i];
    if (part == 1) {
        // s side: A2 = sum_{r>s} dT_rs kr_r e, A4 = sum_{r>=s} dP_rs q_r e
        float kdsum = 0.f;
        for (int s = 0; s < BC; ++s) {
            const float gs = sG[s][i];
            float a2 = 0.f, a4 = 0.f;
            for (int r = s; r < BC; ++r) {
                const float e = __expf(sG[r][i] - gs);
                a2 += sdT[r][s] * sKr[r][i] * e;
                a4 += sdP[r][s] * sQ[r][i] * e;
            }
            const float ed = __expf(Gc - gs);
            const float dkd = DdKd[s * DK + i];
            const float kd = sKw[s][i] * ed;
            kdsum += dkd * kd;
            sW[s][i] = dkd * ed + a2 + a4;
            sDG[s][i] = -dkd * kd - sKw[s][i] * (a2 + a4);
        }
        sDG[BC - 1][i] += kdsum + DdGc[i] * __expf(Gc);
    }
    __syncthreads();
    if (part == 0) {
        // r side: A1 = sum_{s<r} dT_rs kw_s e, A3 = sum_{s<=r} dP_rs kw_s e
        for (int r = 0; r < BC; ++r) {
            const float gr = sG[r][i];
            float a1 = 0.f, a3 = 0.f;
            for (int s = 0; s <= r; ++s) {
                const float wv = sKw[s][i] * __expf(gr - sG[s][i]);
                a1 += sdT[r][s] * wv;
                a3 += sdP[r][s] * wv;
            }
            const float eg = __expf(gr);
            const float dqg = DdQg[r * DK + i], dkg = DdKg[r * DK + i];
            const float dq = dqg * eg + a3;
            const float dkr = dkg * eg + a1;
            const long t = t0 + r;
            if (t < p.T) p.dq[(bh * p.T + t) * DK + i] = dq;
            sDG[r][i] += dkg * sKr[r][i] * eg + dqg * sQ[r][i] * eg + sKr[r][i] * a1 + sQ[r][i] * a3;
            // reuse sKr[r][i] for dkr (only this thread reads it from here on)
            sKr[r][i] = dkr;
        }
        // d log alpha: reverse cumulative sum of dG over the chunk
        float run = 0.f;
        for (int r = BC - 1; r >= 0; --r) {
            run += sDG[r][i];
            const long t = t0 + r;
            const float dla = tok_la_clamped<DK>(p, bh, t, i) ? 0.f : run;
            if (p.amode == PDN_ALPHA_VEC && t < p.T) p.dla[(bh * p.T + t) * DK + i] = dla;
            sDG[r][i] = dla;
        }
        // keys to k and the gains; the preconditioner's dA
        float A = p.pre ? p.apre[(bh * p.nc + c) * DK + i] : 0.f;
        for (int r = 0; r < BC; ++r) {
            const long t = t0 + r;
            const float kk = t < p.T ? ld<BF16>(p.k, (bh * p.T + t) * DK + i) : 0.f;
            const float braw = tok_beta<DK>(p, bh, t, i);
            float b = braw, ainv = 1.f;
            if (p.pre) {
                A += kk * kk;
                ainv = 1.f / (A + p.eps);
                b = braw * ainv;
            }
            const float dkw = sW[r][i], dkr = sKr[r][i];
            float dkk, db;
            if (p.kmode == PDN_KEY_SYMMETRIC) {
                const float sb = sqrtf(b);
                dkk = (dkw + dkr) * sb;
                db = (dkw + dkr) * kk * 0.5f / sb;
            } else if (p.kmode == PDN_KEY_ERASE_GATE) {
                dkk = dkw + dkr * b;
                db = dkr * kk;
            } else {
                dkk = dkw * b + dkr;
                db = dkw * kk;
            }
            float dA = 0.f;
            if (p.pre) {
                dA = -db * braw * ainv * ainv;
                db *= ainv;
            }
            if (p.gmode == PDN_GAMMA_SAME_AS_BETA && p.bmode == PDN_GATE_VEC && t < p.T) {
                // beta also scales the value of column i (dk == dv)
                const float z = p.Z[(bh * Tp + t) * p.dv + i];
                const float vv = ld<BF16>(p.v, (bh * p.T + t) * p.dv + i);
                db += z * vv * value_dscale(p.kmode, p.gmode, braw);
            }
            if (t < p.T) {
                p.dk[(bh * p.T + t) * DK + i] = dkk;
                if (p.bmode == PDN_GATE_VEC) p.dbeta[(bh * p.T + t) * DK + i] = db;
            }
            sW[r][i] = db;
            sQ[r][i] = dA;  // reuse: dA per row
        }
        if (p.pre) {
            float suf = 0.f;
            for (int r = BC - 1; r >= 0; --r) {
                suf += sQ[r][i];
                p.dAin[(bh * Tp + t0 + r) * DK + i] = suf;
            }
            p.dAc[(bh * p.nc + c) * DK + i] = suf;
        }
    }
    __syncthreads();
    // per-token sums for scalar gates
    if (tid < BC) {
        const int r = tid;
        const long t = t0 + r;
        if (t < p.T) {
            if (p.amode == PDN_ALPHA_SCALAR) {
                float s = 0.f;
                for (int ii = 0; ii < DK; ++ii) s += sDG[r][ii];
                p.dla[bh * p.T + t] = s;
            }
            if (p.bmode == PDN_GATE_SCALAR) {
                float s = 0.f;
                for (int ii = 0; ii < DK; ++ii) s += sW[r][ii];
                if (p.gmode == PDN_GAMMA_SAME_AS_BETA) s += sRowG[r];
                p.dbeta[bh * p.T + t] = s;
            }
            if (p.gmode == PDN_GATE_SCALAR) p.dgamma[bh * p.T + t] = sRowG[r];
        }
    }
}

// ---------------------------------------------------------------------------
// preconditioner: dk += 2 k (.) sum_{s >= t} dA_s, dA0
// ---------------------------------------------------------------------------
template <int DK>
__global__ void __launch_bounds__(DK) bwd_dA_scan_kernel(BwdParams p) {
    const long bh = blockIdx.x;
    const int i = threadIdx.x;
    float run = 0.f;
    for (long c = p.nc - 1; c >= 0; --c) {
        p.dAsuf[(bh * p.nc + c) * DK + i] = run;
        run += p.dAc[(bh * p.nc + c) * DK + i];
    }
    if (p.dA0) p.dA0[bh * DK + i] = run;
}

template <int DK, bool BF16>
__global__ void __launch_bounds__(NT) bwd_dA_apply_kernel(BwdParams p) {
    const long bh = blockIdx.x / p.nc;
    const long c = blockIdx.x % p.nc;
    const long Tp = static_cast<long>(p.nc) * BC;
    for (int idx = threadIdx.x; idx < BC * DK; idx += NT) {
        const int r = idx / DK, i = idx % DK;
        const long t = c * BC + r;
        if (t >= p.T) continue;
        const float kk = ld<BF16>(p.k, (bh * p.T + t) * DK + i);
        p.dk[(bh * p.T + t) * DK + i] +=
            2.f * kk * (p.dAin[(bh * Tp + t) * DK + i] + p.dAsuf[(bh * p.nc + c) * DK + i]);
    }
}

// T == 0: dS0 = dST (or 0), dA0 = 0
__global__ void bwd_copy_kernel(float* dst, const float* src, long n) {
    const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct BwdLayout {
    size_t rec, st, dst, U, Z, dgr, apre, ksum, dAin, dAc, dAsuf, end;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

BwdLayout bwd_layout(const pdn_chunk_bwd_args& a) {
    const pdn_chunk_fwd_args& f = a.fwd;
    const size_t nbh = static_cast<size_t>(f.B) * f.H;
    const size_t nc = (static_cast<size_t>(f.T) + BC - 1) / BC;
    const size_t dk = f.dk, dv = f.dv;
    const size_t recf = 3 * BC * dk + 2 * BC * BC + dk + BC * dv;
    const size_t dgrf = 3 * BC * dk + 2 * BC * BC + dk;
    const bool pre = f.precond_eps >= 0.0f;
    BwdLayout L;
    size_t o = 0;
    auto take = [&](size_t floats) {
        const size_t at = o;
        o = align256(o + floats * sizeof(float));
        return at;
    };
    L.rec = take(nbh * nc * recf);
    L.st = take(nbh * (nc + 1) * dk * dv);
    L.dst = take(nbh * nc * dk * dv);
    L.U = take(nbh * nc * BC * dv);
    L.Z = take(nbh * nc * BC * dv);
    L.dgr = take(nbh * nc * dgrf);
    L.apre = take(pre ? nbh * nc * dk : 0);
    L.ksum = take(pre ? nbh * nc * dk : 0);
    L.dAin = take(pre ? nbh * nc * BC * dk : 0);
    L.dAc = take(pre ? nbh * nc * dk : 0);
    L.dAsuf = take(pre ? nbh * nc * dk : 0);
    L.end = o;
    return L;
}

template <int DK, bool BF16>
hipError_t run_bwd(const pdn_chunk_bwd_args& a, const BwdParams& p, hipStream_t s) {
    const unsigned nbh = static_cast<unsigned>(p.nbh);
    const unsigned nch = static_cast<unsigned>(p.nbh * p.nc);
    const unsigned ntl = static_cast<unsigned>(p.nbh * (p.dv / JT));
    (void)a;
    if (p.pre) {
        bwd_ksum_kernel<DK, BF16><<<nch, DK, 0, s>>>(p);
        bwd_kscan_kernel<DK><<<nbh, DK, 0, s>>>(p);
    }
    bwd_prep_kernel<DK, BF16><<<nch, NT, 0, s>>>(p);
    bwd_state_fwd_kernel<DK><<<ntl, NT, 0, s>>>(p);
    bwd_state_bwd_kernel<DK><<<ntl, NT, 0, s>>>(p);
    bwd_dgrad_kernel<DK><<<nch, NT, 0, s>>>(p);
    bwd_gates_kernel<DK, BF16><<<nch, NT, 0, s>>>(p);
    if (p.pre) {
        bwd_dA_scan_kernel<DK><<<nbh, DK, 0, s>>>(p);
        bwd_dA_apply_kernel<DK, BF16><<<nch, NT, 0, s>>>(p);
    }
    return hipGetLastError();
}

}  // namespace

size_t chunk_bwd_workspace_bytes(const pdn_chunk_bwd_args& a) {
    if (a.fwd.T <= 0) return 0;
    return bwd_layout(a).end;
}

hipError_t launch_chunk_bwd(const pdn_chunk_bwd_args& a, hipStream_t stream) {
    const pdn_chunk_fwd_args& f = a.fwd;
    const long nbh = static_cast<long>(f.B) * f.H;
    if (f.T == 0) {
        const long n = nbh * f.dk * f.dv;
        if (a.dS0) bwd_copy_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream>>>(a.dS0, a.dST, n);
        if (a.dA0 && f.precond_eps >= 0.0f)
            bwd_copy_kernel<<<dim3(static_cast<unsigned>((nbh * f.dk + 255) / 256)), dim3(256), 0, stream>>>(
                a.dA0, nullptr, nbh * f.dk);
        return hipGetLastError();
    }
    BwdParams p;
    p.T = f.T;
    p.dv = f.dv;
    p.nc = (f.T + BC - 1) / BC;
    p.nbh = nbh;
    p.q = f.q;
    p.k = f.k;
    p.v = f.v;
    p.amode = f.alpha_mode;
    p.bmode = f.beta_mode;
    p.gmode = f.gamma_mode;
    p.kmode = f.key_mode;
    p.la = f.log_alpha;
    p.beta = f.beta;
    p.gamma = f.gamma;
    p.eps = f.precond_eps;
    p.pre = f.precond_eps >= 0.0f;
    p.A0 = f.precond_A0;
    p.S0 = f.S0;
    p.dO = a.dO;
    p.dST = a.dST;
    p.dq = a.dq;
    p.dk = a.dk;
    p.dvo = a.dv;
    p.dla = a.dlog_alpha;
    p.dbeta = a.dbeta;
    p.dgamma = a.dgamma;
    p.dS0 = a.dS0;
    p.dA0 = a.dA0;
    const BwdLayout L = bwd_layout(a);
    char* ws = static_cast<char*>(a.workspace);
    auto at = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    p.rec = at(L.rec);
    p.st = at(L.st);
    p.dst = at(L.dst);
    p.U = at(L.U);
    p.Z = at(L.Z);
    p.dgr = at(L.dgr);
    p.apre = at(L.apre);
    p.ksum = at(L.ksum);
    p.dAin = at(L.dAin);
    p.dAc = at(L.dAc);
    p.dAsuf = at(L.dAsuf);
    const bool bf = f.qkv_dtype == PDN_BF16;
    if (f.dk == 128) return bf ? run_bwd<128, true>(a, p, stream) : run_bwd<128, false>(a, p, stream);
    return bf ? run_bwd<64, true>(a, p, stream) : run_bwd<64, false>(a, p, stream);
}

}  // namespace pdn
