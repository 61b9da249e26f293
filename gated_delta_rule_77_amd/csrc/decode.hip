// Single-token decode of the gated delta rule against a resident fp32 state.
//
// Per (b,h), with the state S (dk x dv, row i = key channel) read once from
// HBM and written once:
//   A   = Diag(alpha) S                     (alpha = exp(log_alpha))
//   u   = vw - A^T kr
//   p   = A^T q
//   S'  = A + kw u^T
//   o   = S'^T q = p + u (kw . q)
// with the read key kr, write key kw and written value vw of the key mode:
// kr = kw = sqrt(beta') k, vw = sqrt(gamma) v (symmetric); kw = k,
// kr = beta' k, vw = gamma v (erase gate); kw = beta' k, kr = k, vw = v or
// gamma v (write gate).  beta' = beta / (A + eps) with the diagonal
// preconditioner, or beta x^-(r / (1 + |r|)) with r = ln(A + eps) minus its
// mean over the key channels in the stabilised mode (one more block
// reduction per pair).
// Both column reductions over the key channels are taken in the same pass over
// the state, so the state streams through registers exactly once.  This is the
// recurrent (inference) form of the update in "FG^2-GDN" 2.1 / "Gated
// DeltaNet-2" method section 1, with the "Preconditioned DeltaNet" 2.2 running
// diagonal advanced in place when enabled.
//
// Work split: 256-thread workgroups, each walking (b,h) pairs.  Each thread
// owns a float4 column group and DK/NRG rows, so every wave-wide load or store
// covers whole 512-byte (dv = 128) or 256-byte (dv = 64) rows: fully
// coalesced streaming.
#include "common.h"
#include "kernels.h"

namespace pdn {
namespace {

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* gamma;
    float* precond_A;
    float* S;
    void* o;
    float precond_eps;
    float precond_l2x;  // log2 of the stabilised mode's bound x
    int alpha_mode, beta_mode, gamma_mode, key_mode, precond_mode;
};

template <int DK, int DV, bool BF16IN, bool BF16OUT>
__global__ void __launch_bounds__(256, 3) decode_kernel(DecodeParams p, long nbh) {
    constexpr int NCG = DV / 4;       // float4 column groups
    constexpr int NRG = 256 / NCG;    // row groups
    constexpr int RPT = DK / NRG;     // rows per thread
    static_assert(RPT * NRG == DK, "row split");

    const int tid = threadIdx.x;
    const int cg = tid % NCG;
    const int rg = tid / NCG;

    __shared__ float s_alpha[DK], s_kr[DK], s_kw[DK], s_q[DK], s_vw[DV], s_u[DV];
    __shared__ f32x4 s_red[NRG][2][NCG];
    __shared__ float s_kq[4];
    __shared__ float s_mu[2];

    // Persistent workgroups: each walks (b,h) pairs with a stride of the grid
    // and loads the next pair's state while it finishes the current one, so
    // the state stream never stalls on a workgroup's reduction and the grid
    // has no tail.
    auto load_state = [&](long bh, f32x4 (&s)[RPT]) {
        const float* S = p.S + bh * DK * DV;
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            s[m] = *reinterpret_cast<const f32x4*>(S + (long)(rg + NRG * m) * DV + 4 * cg);
    };
    f32x4 s[RPT], sn[RPT];
    long bh = blockIdx.x;
    if (bh < nbh) load_state(bh, s);
    for (; bh < nbh; bh += gridDim.x) {
        const long bn = bh + gridDim.x;
        if (bn < nbh) load_state(bn, sn);
        float* S = p.S + bh * DK * DV;

        // running k (.) k sum and, in the stabilised mode, the coefficient
        // x^-(r / (1 + |r|)), r = ln(A + eps) - mean over the key channels
        const bool pre = p.precond_eps >= 0.0f;
        const bool stab = pre && p.precond_mode == PDN_PRECOND_STABILISED;
        float kk = 0.0f, Aeps = 1.0f, pc = 1.0f;
        if (tid < DK) {
            kk = load_in<BF16IN>(p.k, bh * DK + tid);
            if (pre) {
                const float A = p.precond_A[bh * DK + tid] + kk * kk;
                p.precond_A[bh * DK + tid] = A;
                Aeps = A + p.precond_eps;
            }
        }
        if (stab) {
            const float lg = __builtin_amdgcn_logf(Aeps);  // log2
            if (tid < DK) {
                const float part = wave_sum(lg);
                if ((tid & 63) == 0) s_mu[tid >> 6] = part;
            }
            __syncthreads();
            float mu = s_mu[0];
            if constexpr (DK > 64) mu += s_mu[1];
            const float r = (lg - mu * (1.0f / DK)) * kLn2;
            pc = __builtin_amdgcn_exp2f(-(r / (1.0f + fabsf(r))) * p.precond_l2x);
        }
        if (tid < DK) {
            const int i = tid;
            const float qq = load_in<BF16IN>(p.q, bh * DK + i);
            float la = 0.0f;
            if (p.alpha_mode == PDN_ALPHA_SCALAR) la = p.log_alpha[bh];
            else if (p.alpha_mode == PDN_ALPHA_VEC) la = p.log_alpha[bh * DK + i];
            float b = (p.beta_mode == PDN_GATE_SCALAR) ? p.beta[bh] : p.beta[bh * DK + i];
            if (stab) b = b * pc;
            else if (pre) b = b / Aeps;
            float kr, kw;
            if (p.key_mode == PDN_KEY_ERASE_GATE) {
                kr = b * kk; kw = kk;
            } else if (p.key_mode == PDN_KEY_WRITE_GATE) {
                kr = kk; kw = b * kk;
            } else {
                kr = kw = sqrtf(b) * kk;
            }
            s_alpha[i] = expf(la);
            s_kr[i] = kr;
            s_kw[i] = kw;
            s_q[i] = qq;
            const float part = wave_sum(kw * qq);
            if ((tid & 63) == 0) s_kq[tid >> 6] = part;
        }
        if (tid < DV) {
            const int j = tid;
            float g;
            if (p.gamma_mode == PDN_GAMMA_SAME_AS_BETA)
                g = (p.beta_mode == PDN_GATE_SCALAR) ? p.beta[bh] : p.beta[bh * DK + j];
            else if (p.gamma_mode == PDN_GATE_SCALAR)
                g = p.gamma[bh];
            else
                g = p.gamma[bh * DV + j];
            if (p.key_mode == PDN_KEY_SYMMETRIC) g = sqrtf(g);
            else if (p.key_mode == PDN_KEY_WRITE_GATE && p.gamma_mode == PDN_GAMMA_SAME_AS_BETA) g = 1.0f;
            s_vw[j] = g * load_in<BF16IN>(p.v, bh * DV + j);
        }
        __syncthreads();

        // A = Diag(alpha) S and the two partial column sums over this thread's rows.
        f32x4 u = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int row = rg + NRG * m;
            s[m] *= s_alpha[row];
            u += s[m] * s_kr[row];
            pq += s[m] * s_q[row];
        }
        s_red[rg][0][cg] = u;
        s_red[rg][1][cg] = pq;
        __syncthreads();

        if (tid < DV) {
            const int j = tid;
            float su = 0.0f, sp = 0.0f;
#pragma unroll
            for (int r = 0; r < NRG; ++r) {
                su += s_red[r][0][j >> 2][j & 3];
                sp += s_red[r][1][j >> 2][j & 3];
            }
            float kq = s_kq[0];
            if constexpr (DK > 64) kq += s_kq[1];
            const float uj = s_vw[j] - su;
            const float oj = sp + uj * kq;
            if constexpr (BF16OUT)
                static_cast<uint16_t*>(p.o)[bh * DV + j] = f32_to_bf16_bits(oj);
            else
                static_cast<float*>(p.o)[bh * DV + j] = oj;
            s_u[j] = uj;
        }
        __syncthreads();

        const f32x4 uc = *reinterpret_cast<const f32x4*>(&s_u[4 * cg]);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int row = rg + NRG * m;
            s[m] += s_kw[row] * uc;
            *reinterpret_cast<f32x4*>(S + (long)row * DV + 4 * cg) = s[m];
        }
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = sn[m];
        __syncthreads();  // the shared arrays are rewritten for the next pair
    }
}

template <int DK, int DV>
hipError_t launch_dk_dv(const DecodeParams& p, bool bf16in, bool bf16out, long nbh,
                        hipStream_t st) {
    // exactly the resident workgroups (three per compute unit: the launch
    // bounds keep the kernel within a third of the register file), each
    // walking many (b,h) pairs
    const long resident = 3L * device_cu_count();
    dim3 grid(static_cast<unsigned>(nbh < resident ? nbh : resident)), block(256);
    if (bf16in && bf16out) decode_kernel<DK, DV, true, true><<<grid, block, 0, st>>>(p, nbh);
    else if (bf16in) decode_kernel<DK, DV, true, false><<<grid, block, 0, st>>>(p, nbh);
    else if (bf16out) decode_kernel<DK, DV, false, true><<<grid, block, 0, st>>>(p, nbh);
    else decode_kernel<DK, DV, false, false><<<grid, block, 0, st>>>(p, nbh);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const pdn_decode_args& a, hipStream_t stream) {
    DecodeParams p;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.log_alpha = a.log_alpha; p.beta = a.beta; p.gamma = a.gamma;
    p.precond_A = a.precond_A; p.S = a.S; p.o = a.o;
    p.precond_eps = a.precond_eps;
    p.precond_mode = a.precond_mode;
    p.precond_l2x = a.precond_mode == PDN_PRECOND_STABILISED ? std::log2(a.precond_x) : 0.0f;
    p.alpha_mode = a.alpha_mode; p.beta_mode = a.beta_mode; p.gamma_mode = a.gamma_mode;
    p.key_mode = a.key_mode;
    const long nbh = static_cast<long>(a.B) * a.H;
    const bool bi = a.qkv_dtype == PDN_BF16, bo = a.o_dtype == PDN_BF16;
    if (a.dk == 128 && a.dv == 128) return launch_dk_dv<128, 128>(p, bi, bo, nbh, stream);
    if (a.dk == 128 && a.dv == 64) return launch_dk_dv<128, 64>(p, bi, bo, nbh, stream);
    if (a.dk == 64 && a.dv == 128) return launch_dk_dv<64, 128>(p, bi, bo, nbh, stream);
    return launch_dk_dv<64, 64>(p, bi, bo, nbh, stream);
}

}  // namespace pdn
