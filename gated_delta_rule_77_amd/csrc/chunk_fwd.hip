// Chunkwise-parallel prefill of the gated delta rule on gfx950.
//
// Algorithm (chunk form of the recurrence; "Gated DeltaNet-2" method section 3
// absorbs the cumulative decay into the erase/write matrices and solves a
// unit-lower-triangular (I+T) system per chunk; "FG^2-GDN" 2.3 notes the
// diagonal-plus-low-rank transition that makes this possible).  For a block of
// 16 tokens r = 0..15 starting from state S (dk x dv), with G_r the cumulative
// log-decay inside the block (per key channel), Gamma_r = exp(G_r),
// kt_r = sqrt(beta'_r) k_r and vt_r = sqrt(gamma_r) v_r:
//
//   T_rs = sum_i kt_ri kt_si exp(G_ri - G_si)          s < r   (16 x 16)
//   P_rs = sum_i q_ri  kt_si exp(G_ri - G_si)          s <= r
//   U    = (I + T)^-1 (Vt - (Kt . Gamma) S)
//   O    = (Q . Gamma) S + P U
//   S   <- Diag(Gamma_15) S + (Kt . exp(G_15 - G))^T U
//
// which reproduces the token recurrence exactly in exact arithmetic.
//
// Mapping to the GPU.  One workgroup per (b, h, dv tile of 16*NW columns);
// wave w owns 16 columns of S for the whole sequence, held in MFMA
// accumulator layout in registers.  Tokens stream in 64-token load chunks:
//   phase A (whole workgroup): stage the chunk in LDS, form the gate
//     quantities, the four 16x16 T and P blocks (MFMA) and the four
//     (I+T)^-1 blocks (forward substitution, one lane per column);
//   phase B (each wave on its own columns, no barriers): four 16-token
//     state updates, each KS/QS (16x16x32 MFMA over dk), the 16x16 solve,
//     the output, and the rank-16 state update (16x16x16 MFMA).
// The next chunk's global loads are issued before phase B and land in
// registers while phase B runs.
//
// Precision.  q/k/v in bf16 enter the MFMAs unchanged (exact).  Every derived
// operand (state, solve blocks, gate-scaled keys/queries, U) is split into
// bf16 hi + lo terms (three terms on the fp32-input path) and the products of
// the terms that matter are accumulated in fp32, giving ~16-bit (fp32 path:
// ~24-bit) operands at bf16 MFMA rate.  The state is kept in fp32.
//
// Two gate paths:
//   FACTORED (decay and erase gain scalar per token, no preconditioner): the
//     gates factor out of every dot product, so raw q/k feed the MFMAs and the
//     gates are applied as fp32 row scales.
//   VEC (any per-channel decay or gain, or the preconditioner): gate-scaled
//     operands are formed per element in LDS.  exp(G_r - G_s) inside a block
//     is split around the block's middle token; the per-token clamp of
//     log(alpha) at -10 keeps both factors in range.
#include "common.h"
#include "kernels.h"

namespace pdn {
namespace {

constexpr int CH = 64;             // tokens per load chunk
constexpr int NSB = 4;             // 16-token blocks per chunk
constexpr int BLKP = 20;           // row stride (floats) of a 16x16 block buffer
constexpr int BLKS = 16 * BLKP + 16;  // stride between the four block buffers

struct ChunkParams {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* A0;
    float* AT;
    const float* S0;
    float* ST;
    void* o;
    const float* gsrc;  // value-side gain source: gamma, or beta when "same as beta"
    long gts;           // its stride per token (elements)
    long T;
    int dv;
    int alpha_mode, beta_mode;
    int gvec;           // value gain is per column (else one scalar per token)
    float eps;          // < 0: preconditioner off
    int o_bf16;
};

// ---------------------------------------------------------------------------
// layout helpers
// ---------------------------------------------------------------------------

// Physical column of logical column k in a "k-permuted" row: inside every
// 32-column group the 4-column groups are interleaved so that one 16-byte read
// per lane yields the eight MFMA k-slots {4g..4g+3, 16+4g..16+4g+3}, which is
// the order in which two stacked 16x16 accumulator tiles hold their rows.
__device__ __forceinline__ int perm_col(int k) {
    const int q = k >> 2;
    const int pq = (q & ~7) | ((q & 3) << 1) | ((q >> 2) & 1);
    return (pq << 2) | (k & 3);
}
__device__ __forceinline__ int unperm_col(int pc) {
    const int pq = pc >> 2;
    const int q = (pq & ~7) | ((pq & 1) << 2) | ((pq >> 1) & 3);
    return (q << 2) | (pc & 3);
}

template <bool F32IN>
struct Raw;
template <>
struct Raw<false> {
    using T = uint16_t;
    static constexpr int PIECE = 8;  // elements per 16-byte piece
    static constexpr int PAD = 8;
    static constexpr int NT = 1;     // bf16 terms of a raw operand
};
template <>
struct Raw<true> {
    using T = float;
    static constexpr int PIECE = 4;
    static constexpr int PAD = 4;
    static constexpr int NT = 3;
};

template <int DK, int NW, bool F32IN, bool VEC>
struct Cfg {
    using R = Raw<F32IN>;
    using RawT = typename R::T;
    static constexpr int NTHR = 64 * NW;
    static constexpr int DVT = 16 * NW;
    static constexpr int NTR = R::NT;                 // terms of raw operands
    static constexpr int NTD = F32IN ? 3 : 2;         // terms of derived operands
    static constexpr int RS = DK + R::PAD;            // raw [64][DK] row stride
    static constexpr int FS = DK + 4;                 // fp32 [64][DK] row stride
    static constexpr int VS = DVT + 4;                // fp32 V tile row stride
    static constexpr int CT = CH + R::PAD;            // raw K^T row stride (FACTORED)
    static constexpr int ES = CH + 4;                 // fp32 Khat^T row stride (VEC)
    static constexpr int KPC = 64 * DK / R::PIECE;    // raw pieces per chunk
    static constexpr int KP = KPC / NTHR;             // raw pieces per thread
    static constexpr int VPC = 64 * DVT / R::PIECE;
    static constexpr int VP = VPC / NTHR;
    static constexpr int GP = 64 * DK / 4 / NTHR;     // fp32 gate pieces per thread (VEC)
    static_assert(KP * NTHR == KPC && VP * NTHR == VPC && GP * NTHR * 4 == 64 * DK, "split");

    static constexpr int RAWB = 64 * RS * (int)sizeof(RawT);
    static constexpr int F32B = 64 * FS * 4;
    static constexpr int VB = 64 * VS * 4;
    static constexpr int BLKB = NSB * BLKS * 4;
    // FACTORED layout
    static constexpr int F_K = 0;
    static constexpr int F_Q = F_K + RAWB;
    static constexpr int F_KT = F_Q + RAWB;
    static constexpr int F_V = F_KT + DK * CT * (int)sizeof(RawT);
    static constexpr int F_T = F_V + VB;
    static constexpr int F_P = F_T + BLKB;
    static constexpr int F_SC = F_P + BLKB;            // 6 x 64 floats of per-token scalars
    static constexpr int F_END = F_SC + 6 * 64 * 4 + 16 * 4;
    // VEC layout
    static constexpr int EB = (DK * ES * 4 > RAWB) ? DK * ES * 4 : RAWB;
    static constexpr int V_A = 0;                      // beta -> Kt -> Kt.Gamma
    static constexpr int V_B = V_A + F32B;             // log alpha -> G2 -> Q.Gamma
    static constexpr int V_Q = V_B + F32B;             // raw q
    static constexpr int V_E = V_Q + RAWB;             // raw k -> Khat^T
    static constexpr int V_V = V_E + EB;
    static constexpr int V_T = V_V + VB;
    static constexpr int V_P = V_T + BLKB;
    static constexpr int V_GC = V_P + BLKB;            // [NSB][DK] block-end decay
    static constexpr int V_AC = V_GC + NSB * DK * 4;   // [DK] preconditioner carry
    static constexpr int V_BS = V_AC + DK * 4;         // [NSB][DK] block sums of k*k
    static constexpr int V_END = V_BS + NSB * DK * 4;
    static constexpr int LDS = VEC ? V_END : F_END;
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// ---------------------------------------------------------------------------
// operand helpers
// ---------------------------------------------------------------------------

template <int NT, int N>
__device__ __forceinline__ void split_terms(const float* x, bf16 (&o)[NT][N]) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
        float r = x[e];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bf16 h = static_cast<bf16>(r);
            o[t][e] = h;
            if (t + 1 < NT) r -= static_cast<float>(h);
        }
    }
}

template <int NT>
__device__ __forceinline__ void split8(const float* x, bf16x8 (&o)[NT]) {
    bf16 tmp[NT][8];
    split_terms<NT, 8>(x, tmp);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[t][e] = tmp[t][e];
}

template <int NT>
__device__ __forceinline__ void split4(const float* x, bf16x4 (&o)[NT]) {
    bf16 tmp[NT][4];
    split_terms<NT, 4>(x, tmp);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[t][e] = tmp[t][e];
}

// acc += sum over term pairs (i, j) with i + j < max(NA, NB) of a_i b_j,
// smallest terms first.
template <int NA, int NB>
__device__ __forceinline__ void mma32(f32x4& acc, const bf16x8 (&a)[NA], const bf16x8 (&b)[NB]) {
    constexpr int N = NA > NB ? NA : NB;
#pragma unroll
    for (int s = N - 1; s >= 0; --s)
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int j = s - i;
            if (j >= 0 && j < NB)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc, 0, 0, 0);
        }
}

template <int NA, int NB>
__device__ __forceinline__ void mma16(f32x4& acc, const bf16x4 (&a)[NA], const bf16x4 (&b)[NB]) {
    constexpr int N = NA > NB ? NA : NB;
#pragma unroll
    for (int s = N - 1; s >= 0; --s)
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int j = s - i;
            if (j >= 0 && j < NB)
                acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[i], b[j], acc, 0, 0, 0);
        }
}

// 8 consecutive elements of a raw [.][.] LDS buffer as an x32 MFMA operand.
template <bool F32IN>
__device__ __forceinline__ void raw_op8(const typename Raw<F32IN>::T* p,
                                        bf16x8 (&o)[Raw<F32IN>::NT]) {
    if constexpr (!F32IN) {
        o[0] = *reinterpret_cast<const bf16x8*>(p);
    } else {
        float x[8];
        *reinterpret_cast<f32x4*>(x) = *reinterpret_cast<const f32x4*>(p);
        *reinterpret_cast<f32x4*>(x + 4) = *reinterpret_cast<const f32x4*>(p + 4);
        split8<3>(x, o);
    }
}

// 4 consecutive elements of a raw LDS buffer as an x16 MFMA operand.
template <bool F32IN>
__device__ __forceinline__ void raw_op4(const typename Raw<F32IN>::T* p,
                                        bf16x4 (&o)[Raw<F32IN>::NT]) {
    if constexpr (!F32IN) {
        o[0] = *reinterpret_cast<const bf16x4*>(p);
    } else {
        float x[4];
        *reinterpret_cast<f32x4*>(x) = *reinterpret_cast<const f32x4*>(p);
        split4<3>(x, o);
    }
}

template <int NT>
__device__ __forceinline__ void f32_op8(const float* p, bf16x8 (&o)[NT]) {
    float x[8];
    *reinterpret_cast<f32x4*>(x) = *reinterpret_cast<const f32x4*>(p);
    *reinterpret_cast<f32x4*>(x + 4) = *reinterpret_cast<const f32x4*>(p + 4);
    split8<NT>(x, o);
}

template <int NT>
__device__ __forceinline__ void f32_op4(const float* p, bf16x4 (&o)[NT]) {
    float x[4];
    *reinterpret_cast<f32x4*>(x) = *reinterpret_cast<const f32x4*>(p);
    split4<NT>(x, o);
}

__device__ __forceinline__ float raw_to_f32(uint16_t b) { return bf16_bits_to_f32(b); }
__device__ __forceinline__ float raw_to_f32(float x) { return x; }

__device__ __forceinline__ float clamp_log_alpha(float la) {
    return fmaxf(la, kLogAlphaMin) * kLog2e;  // natural log -> log2 units
}

// Forward substitution for the four 16x16 unit-lower-triangular blocks held
// in-place in `blk` (T in, (I+T)^-1 out).  One wave; lane = (block, column).
__device__ __forceinline__ void invert_blocks(float* blk, int lane) {
    float* B = blk + (lane >> 4) * BLKS;
    const int c = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.0f : 0.0f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < r; ++j) acc = fmaf(B[r * BLKP + j], x[j], acc);
        if (r > c) x[r] = -acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) B[r * BLKP + c] = x[r];
}

// ---------------------------------------------------------------------------
// global -> register prefetch of one 64-token chunk
// ---------------------------------------------------------------------------

template <int DK, int NW, bool F32IN, bool VEC>
struct Stage {
    using C = Cfg<DK, NW, F32IN, VEC>;
    uint4 k[C::KP];
    uint4 q[C::KP];
    uint4 v[C::VP];
    f32x4 gam[C::VP * Raw<F32IN>::PIECE / 4];  // per-column value gain
    float gam1[C::VP];                          // or one value gain per token
    f32x4 la[VEC ? C::GP : 1];                  // per-channel log decay
    f32x4 be[VEC ? C::GP : 1];                  // per-channel gain
    float la1[VEC ? C::GP : 1];                 // or one value per token
    float be1[VEC ? C::GP : 1];
    float fla, fbe;  // FACTORED: per-token scalars (threads < 64)
};

// Loads are unconditional: rows past the end of the sequence read the last
// valid token (always in bounds) and are zeroed when staged into LDS.  No
// loaded value is touched here, so the loads stay in flight until staging.
template <int DK, int NW, bool F32IN, bool VEC>
__device__ __forceinline__ void prefetch(Stage<DK, NW, F32IN, VEC>& st, const ChunkParams& p,
                                         long bh, long t0, int j0, int tid) {
    using C = Cfg<DK, NW, F32IN, VEC>;
    using RawT = typename C::RawT;
    constexpr int PIECE = Raw<F32IN>::PIECE;
    constexpr int PPR = DK / PIECE;  // pieces per row
    const long tmax = p.T - 1;
    const RawT* K = static_cast<const RawT*>(p.k);
    const RawT* Q = static_cast<const RawT*>(p.q);
    const RawT* V = static_cast<const RawT*>(p.v);
#pragma unroll
    for (int m = 0; m < C::KP; ++m) {
        const int pi = tid + m * C::NTHR;
        const int row = pi / PPR, col = (pi % PPR) * PIECE;
        const long t = min(t0 + row, tmax);
        const long off = (bh * p.T + t) * DK + col;
        st.k[m] = *reinterpret_cast<const uint4*>(K + off);
        st.q[m] = *reinterpret_cast<const uint4*>(Q + off);
    }
    constexpr int VPR = C::DVT / PIECE;
#pragma unroll
    for (int m = 0; m < C::VP; ++m) {
        const int pi = tid + m * C::NTHR;
        const int row = pi / VPR, col = (pi % VPR) * PIECE;
        const long tok = bh * p.T + min(t0 + row, tmax);
        st.v[m] = *reinterpret_cast<const uint4*>(V + tok * p.dv + j0 + col);
        if (p.gvec) {
#pragma unroll
            for (int h = 0; h < PIECE / 4; ++h)
                st.gam[m * (PIECE / 4) + h] =
                    *reinterpret_cast<const f32x4*>(p.gsrc + tok * p.gts + j0 + col + 4 * h);
        } else {
            st.gam1[m] = p.gsrc[tok * p.gts];
        }
    }
    if constexpr (VEC) {
        constexpr int GPR = DK / 4;
#pragma unroll
        for (int m = 0; m < C::GP; ++m) {
            const int pi = tid + m * C::NTHR;
            const int row = pi / GPR, col = (pi % GPR) * 4;
            const long tok = bh * p.T + min(t0 + row, tmax);
            if (p.alpha_mode == PDN_ALPHA_VEC)
                st.la[m] = *reinterpret_cast<const f32x4*>(p.log_alpha + tok * DK + col);
            else if (p.alpha_mode == PDN_ALPHA_SCALAR)
                st.la1[m] = p.log_alpha[tok];
            if (p.beta_mode == PDN_GATE_VEC)
                st.be[m] = *reinterpret_cast<const f32x4*>(p.beta + tok * DK + col);
            else
                st.be1[m] = p.beta[tok];
        }
    } else {
        if (tid < CH) {
            const long tok = bh * p.T + min(t0 + tid, tmax);
            if (p.alpha_mode != PDN_ALPHA_NONE) st.fla = p.log_alpha[tok];
            st.fbe = p.beta[tok];
        }
    }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

template <int DK, int NW, bool F32IN, bool VEC>
__global__ void __launch_bounds__(64 * NW) chunk_fwd_kernel(ChunkParams p) {
    using C = Cfg<DK, NW, F32IN, VEC>;
    using RawT = typename C::RawT;
    constexpr int NTR = C::NTR, NTD = C::NTD;
    constexpr int PIECE = Raw<F32IN>::PIECE;
    constexpr int NKT = DK / 32;   // x32 k-steps over dk
    constexpr int NIB = DK / 16;   // 16-row tiles of S

    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;       // lane group (MFMA k/row quad)
    const int ln = lane & 15;      // lane within group
    const int ntile = p.dv / C::DVT;
    const long bh = blockIdx.x / ntile;
    const int tile = blockIdx.x % ntile;
    const int j0 = tile * C::DVT;          // first value column of this workgroup
    const int col = j0 + 16 * wave + ln;   // this lane's value column
    const long nchunks = (p.T + CH - 1) / CH;
    const bool precond = VEC && p.eps >= 0.0f;

    // ---- state: S[16*ib + 4g + e][col] in sacc[ib][e] ----
    f32x4 sacc[NIB];
    if (p.S0) {
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sacc[ib][e] = p.S0[(bh * DK + 16 * ib + 4 * g + e) * p.dv + col];
    } else {
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) sacc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if constexpr (VEC) {
        float* Ac = reinterpret_cast<float*>(smem + C::V_AC);
        // the carry is indexed by physical (permuted) channel, like the gate buffers
        for (int pc = tid; pc < DK; pc += C::NTHR)
            Ac[pc] = p.A0 ? p.A0[bh * DK + unperm_col(pc)] : 0.0f;
    }

    Stage<DK, NW, F32IN, VEC> st;
    if (nchunks > 0) prefetch<DK, NW, F32IN, VEC>(st, p, bh, 0, j0, tid);

    for (long c = 0; c < nchunks; ++c) {
        const long t0 = c * CH;
        __syncthreads();  // previous chunk's phase B is done with LDS

        // ================= phase A1: stage raw data in LDS =================
        {
            constexpr int PPR = DK / PIECE;
            RawT* sK = reinterpret_cast<RawT*>(smem + (VEC ? C::V_E : C::F_K));
            RawT* sQ = reinterpret_cast<RawT*>(smem + (VEC ? C::V_Q : C::F_Q));
#pragma unroll
            for (int m = 0; m < C::KP; ++m) {
                const int pi = tid + m * C::NTHR;
                const int row = pi / PPR, c0 = (pi % PPR) * PIECE;
                if (t0 + row >= p.T) {
                    st.k[m] = uint4{0u, 0u, 0u, 0u};
                    st.q[m] = uint4{0u, 0u, 0u, 0u};
                }
                // write PIECE logical columns as 4-column groups at permuted spots
#pragma unroll
                for (int h = 0; h < PIECE / 4; ++h) {
                    const int pc = perm_col(c0 + 4 * h);
                    if constexpr (F32IN) {
                        *reinterpret_cast<uint4*>(sK + row * C::RS + pc) = st.k[m];
                        *reinterpret_cast<uint4*>(sQ + row * C::RS + pc) = st.q[m];
                    } else {
                        const uint2 kk = h ? uint2{st.k[m].z, st.k[m].w} : uint2{st.k[m].x, st.k[m].y};
                        const uint2 qq = h ? uint2{st.q[m].z, st.q[m].w} : uint2{st.q[m].x, st.q[m].y};
                        *reinterpret_cast<uint2*>(sK + row * C::RS + pc) = kk;
                        *reinterpret_cast<uint2*>(sQ + row * C::RS + pc) = qq;
                    }
                }
                if constexpr (!VEC) {  // transposed raw keys for the state update
                    RawT* sKT = reinterpret_cast<RawT*>(smem + C::F_KT);
                    const RawT* ke = reinterpret_cast<const RawT*>(&st.k[m]);
#pragma unroll
                    for (int e = 0; e < PIECE; ++e) sKT[(c0 + e) * C::CT + row] = ke[e];
                }
            }
            // value tile, scaled by sqrt(gamma)
            float* sV = reinterpret_cast<float*>(smem + (VEC ? C::V_V : C::F_V));
            constexpr int VPR = C::DVT / PIECE;
#pragma unroll
            for (int m = 0; m < C::VP; ++m) {
                const int pi = tid + m * C::NTHR;
                const int row = pi / VPR, c0 = (pi % VPR) * PIECE;
                const bool ok = t0 + row < p.T;
                const RawT* ve = reinterpret_cast<const RawT*>(&st.v[m]);
#pragma unroll
                for (int h = 0; h < PIECE / 4; ++h) {
                    f32x4 gm;
                    if (p.gvec) gm = st.gam[m * (PIECE / 4) + h];
                    else gm = f32x4{st.gam1[m], st.gam1[m], st.gam1[m], st.gam1[m]};
                    f32x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        out[e] = ok ? sqrtf(gm[e]) * raw_to_f32(ve[4 * h + e]) : 0.0f;
                    *reinterpret_cast<f32x4*>(sV + row * C::VS + c0 + 4 * h) = out;
                }
            }
            if constexpr (VEC) {
                float* sA = reinterpret_cast<float*>(smem + C::V_A);
                float* sB = reinterpret_cast<float*>(smem + C::V_B);
                constexpr int GPR = DK / 4;
#pragma unroll
                for (int m = 0; m < C::GP; ++m) {
                    const int pi = tid + m * C::NTHR;
                    const int row = pi / GPR, pc = perm_col((pi % GPR) * 4);
                    const bool ok = t0 + row < p.T;
                    f32x4 be = (p.beta_mode == PDN_GATE_VEC)
                                   ? st.be[m]
                                   : f32x4{st.be1[m], st.be1[m], st.be1[m], st.be1[m]};
                    f32x4 la = {0.f, 0.f, 0.f, 0.f};
                    if (p.alpha_mode == PDN_ALPHA_VEC) la = st.la[m];
                    else if (p.alpha_mode == PDN_ALPHA_SCALAR)
                        la = f32x4{st.la1[m], st.la1[m], st.la1[m], st.la1[m]};
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    *reinterpret_cast<f32x4*>(sA + row * C::FS + pc) = ok ? be : zero;
                    *reinterpret_cast<f32x4*>(sB + row * C::FS + pc) = ok ? la : zero;
                }
            } else {
                // per-token scalars: block-relative cumulative decay (log2 units)
                float* sc = reinterpret_cast<float*>(smem + C::F_SC);
                if (tid < CH) {
                    const bool ok = t0 + tid < p.T;
                    float gl = clamp_log_alpha(st.fla);
                    if (p.alpha_mode == PDN_ALPHA_NONE || !ok) gl = 0.0f;
                    const float fbe = ok ? st.fbe : 0.0f;
#pragma unroll
                    for (int d = 1; d < 16; d <<= 1) {
                        const float o = __shfl_up(gl, d, 16);
                        if ((tid & 15) >= d) gl += o;
                    }
                    const float last = __shfl(gl, (tid & ~15) + 15, 64);
                    const float sb = sqrtf(fbe);
                    sc[0 * CH + tid] = gl;                          // G2
                    sc[1 * CH + tid] = sb;                          // sqrt(beta)
                    sc[2 * CH + tid] = sb * exp2f(gl);              // rows of K.Gamma
                    sc[3 * CH + tid] = exp2f(gl);                   // rows of Q.Gamma
                    sc[4 * CH + tid] = sb * exp2f(last - gl);       // rows of Khat
                    if ((tid & 15) == 15) sc[6 * CH + (tid >> 4)] = exp2f(last);  // block decay
                }
            }
        }
        __syncthreads();

        if constexpr (VEC) {
            // ============ phase A2 (VEC): per-channel gate pass ============
            float* sA = reinterpret_cast<float*>(smem + C::V_A);   // beta -> Kt
            float* sB = reinterpret_cast<float*>(smem + C::V_B);   // log alpha -> G2
            const RawT* sK = reinterpret_cast<const RawT*>(smem + C::V_E);
            float* gC = reinterpret_cast<float*>(smem + C::V_GC);
            float* Ac = reinterpret_cast<float*>(smem + C::V_AC);
            float* Bs = reinterpret_cast<float*>(smem + C::V_BS);
            constexpr int NPAIR = DK * NSB;
            if (precond) {
                for (int pr = tid; pr < NPAIR; pr += C::NTHR) {
                    const int pc = pr % DK, jb = pr / DK;
                    float s = 0.0f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float kk = raw_to_f32(sK[(16 * jb + r) * C::RS + pc]);
                        s = fmaf(kk, kk, s);
                    }
                    Bs[jb * DK + pc] = s;
                }
                __syncthreads();
            }
            for (int pr = tid; pr < NPAIR; pr += C::NTHR) {
                const int pc = pr % DK, jb = pr / DK;
                float carry = 0.0f;
                if (precond) {
                    carry = Ac[pc];
                    for (int b2 = 0; b2 < jb; ++b2) carry += Bs[b2 * DK + pc];
                }
                float G = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int idx = (16 * jb + r) * C::FS + pc;
                    if (p.alpha_mode != PDN_ALPHA_NONE) G += clamp_log_alpha(sB[idx]);
                    sB[idx] = G;
                    const float kk = raw_to_f32(sK[(16 * jb + r) * C::RS + pc]);
                    float b = sA[idx];
                    if (precond) {
                        carry = fmaf(kk, kk, carry);
                        b = b / (carry + p.eps);
                    }
                    sA[idx] = sqrtf(b) * kk;
                }
                gC[jb * DK + unperm_col(pc)] = exp2f(G);
            }
            __syncthreads();
            if (precond) {
                for (int pc = tid; pc < DK; pc += C::NTHR) {
                    float s = Ac[pc];
#pragma unroll
                    for (int b2 = 0; b2 < NSB; ++b2) s += Bs[b2 * DK + pc];
                    Ac[pc] = s;
                }
            }

            // ============ phase A3 (VEC): T and P blocks ============
            {
                const RawT* sQ = reinterpret_cast<const RawT*>(smem + C::V_Q);
                float* sT = reinterpret_cast<float*>(smem + C::V_T);
                float* sP = reinterpret_cast<float*>(smem + C::V_P);
                for (int jb = wave; jb < NSB; jb += NW) {
                    const int row = 16 * jb + ln;
                    const int ref = 16 * jb + 7;
                    f32x4 accT = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < NKT; ++t) {
                        const int pc0 = 32 * t + 8 * g;
                        float lk[8], lq[8], rk[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float d = sB[row * C::FS + pc0 + e] - sB[ref * C::FS + pc0 + e];
                            const float kt = sA[row * C::FS + pc0 + e];
                            const float up = exp2f(d), dn = exp2f(-d);
                            lk[e] = kt * up;
                            lq[e] = raw_to_f32(sQ[row * C::RS + pc0 + e]) * up;
                            rk[e] = kt * dn;
                        }
                        bf16x8 aK[NTD], aQ[NTD], bR[NTD];
                        split8<NTD>(lk, aK);
                        split8<NTD>(lq, aQ);
                        split8<NTD>(rk, bR);
                        mma32<NTD, NTD>(accT, aK, bR);
                        mma32<NTD, NTD>(accP, aQ, bR);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g + e, s = ln;
                        sT[jb * BLKS + r * BLKP + s] = (s < r) ? accT[e] : 0.0f;
                        sP[jb * BLKS + r * BLKP + s] = (s <= r) ? accP[e] : 0.0f;
                    }
                }
            }
            __syncthreads();

            // ==== phase A4 (VEC): (I+T)^-1 blocks (wave 0); Khat^T (all) ====
            {
                if (wave == 0) invert_blocks(reinterpret_cast<float*>(smem + C::V_T), lane);
                float* sE = reinterpret_cast<float*>(smem + C::V_E);  // raw k no longer needed
                for (int idx = tid; idx < CH * DK; idx += C::NTHR) {
                    const int r = idx / DK, pc = idx % DK;
                    const int last = (r & ~15) + 15;
                    const float f = exp2f(sB[last * C::FS + pc] - sB[r * C::FS + pc]);
                    sE[unperm_col(pc) * C::ES + r] = sA[r * C::FS + pc] * f;
                }
            }
            __syncthreads();
            // ==== phase A5 (VEC): in place Kt -> Kt.Gamma, G2 -> Q.Gamma ====
            {
                const RawT* sQ = reinterpret_cast<const RawT*>(smem + C::V_Q);
                for (int idx = tid; idx < CH * DK; idx += C::NTHR) {
                    const int r = idx / DK, pc = idx % DK;
                    const float gm = exp2f(sB[r * C::FS + pc]);
                    sA[r * C::FS + pc] *= gm;
                    sB[r * C::FS + pc] = raw_to_f32(sQ[r * C::RS + pc]) * gm;
                }
            }
            __syncthreads();
        } else {
            // ============ phase A2 (FACTORED): T and P blocks ============
            {
                const RawT* sK = reinterpret_cast<const RawT*>(smem + C::F_K);
                const RawT* sQ = reinterpret_cast<const RawT*>(smem + C::F_Q);
                const float* sc = reinterpret_cast<const float*>(smem + C::F_SC);
                float* sT = reinterpret_cast<float*>(smem + C::F_T);
                float* sP = reinterpret_cast<float*>(smem + C::F_P);
                for (int jb = wave; jb < NSB; jb += NW) {
                    const int row = 16 * jb + ln;
                    f32x4 accT = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < NKT; ++t) {
                        const int pc0 = 32 * t + 8 * g;
                        bf16x8 aK[NTR], aQ[NTR];
                        raw_op8<F32IN>(sK + row * C::RS + pc0, aK);
                        raw_op8<F32IN>(sQ + row * C::RS + pc0, aQ);
                        mma32<NTR, NTR>(accT, aK, aK);
                        mma32<NTR, NTR>(accP, aQ, aK);
                    }
                    const int s = ln;
                    const float Gs = sc[16 * jb + s], sbs = sc[CH + 16 * jb + s];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g + e;
                        const float Gr = sc[16 * jb + r], sbr = sc[CH + 16 * jb + r];
                        const float dec = exp2f(Gr - Gs);
                        sT[jb * BLKS + r * BLKP + s] = (s < r) ? accT[e] * sbr * sbs * dec : 0.0f;
                        sP[jb * BLKS + r * BLKP + s] = (s <= r) ? accP[e] * sbs * dec : 0.0f;
                    }
                }
            }
            __syncthreads();
            if (wave == 0) invert_blocks(reinterpret_cast<float*>(smem + C::F_T), lane);
            __syncthreads();
        }

        // prefetch the next chunk while phase B runs
        if (c + 1 < nchunks) prefetch<DK, NW, F32IN, VEC>(st, p, bh, t0 + CH, j0, tid);

        // ================= phase B: per-wave state updates =================
        {
            const float* sV = reinterpret_cast<const float*>(smem + (VEC ? C::V_V : C::F_V));
            const float* sD = reinterpret_cast<const float*>(smem + (VEC ? C::V_T : C::F_T));
            const float* sP = reinterpret_cast<const float*>(smem + (VEC ? C::V_P : C::F_P));
            const int vcol = 16 * wave + ln;  // column inside the tile
#pragma unroll 1
            for (int jb = 0; jb < NSB; ++jb) {
                // state as B operand of the x32 products (k = key channel)
                bf16x8 bS[NKT][NTD];
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = sacc[2 * t][e];
                        x[4 + e] = sacc[2 * t + 1][e];
                    }
                    split8<NTD>(x, bS[t]);
                }
                // Y = (K.Gamma) S  and  Z = (Q.Gamma) S  for this block's 16 rows
                f32x4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
                const int row = 16 * jb + ln;
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    const int pc0 = 32 * t + 8 * g;
                    if constexpr (VEC) {
                        const float* sA = reinterpret_cast<const float*>(smem + C::V_A);
                        const float* sB = reinterpret_cast<const float*>(smem + C::V_B);
                        bf16x8 aK[NTD], aQ[NTD];
                        f32_op8<NTD>(sA + row * C::FS + pc0, aK);
                        f32_op8<NTD>(sB + row * C::FS + pc0, aQ);
                        mma32<NTD, NTD>(y, aK, bS[t]);
                        mma32<NTD, NTD>(z, aQ, bS[t]);
                    } else {
                        const RawT* sK = reinterpret_cast<const RawT*>(smem + C::F_K);
                        const RawT* sQ = reinterpret_cast<const RawT*>(smem + C::F_Q);
                        bf16x8 aK[NTR], aQ[NTR];
                        raw_op8<F32IN>(sK + row * C::RS + pc0, aK);
                        raw_op8<F32IN>(sQ + row * C::RS + pc0, aQ);
                        mma32<NTR, NTD>(y, aK, bS[t]);
                        mma32<NTR, NTD>(z, aQ, bS[t]);
                    }
                }
                // X = Vt - (K.Gamma) S
                float xv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * jb + 4 * g + e;
                    float yy = y[e];
                    if constexpr (!VEC) yy *= reinterpret_cast<const float*>(smem + C::F_SC)[2 * CH + r];
                    xv[e] = sV[r * C::VS + vcol] - yy;
                }
                // U = (I+T)^-1 X
                bf16x4 bX[NTD], aD[NTD];
                split4<NTD>(xv, bX);
                f32_op4<NTD>(sD + jb * BLKS + ln * BLKP + 4 * g, aD);
                f32x4 u = {0.f, 0.f, 0.f, 0.f};
                mma16<NTD, NTD>(u, aD, bX);
                // O = (Q.Gamma) S + P U
                float uv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) uv[e] = u[e];
                bf16x4 bU[NTD], aP[NTD];
                split4<NTD>(uv, bU);
                f32_op4<NTD>(sP + jb * BLKS + ln * BLKP + 4 * g, aP);
                f32x4 oacc = z;
                if constexpr (!VEC) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        oacc[e] *= reinterpret_cast<const float*>(smem + C::F_SC)[3 * CH + 16 * jb + 4 * g + e];
                }
                mma16<NTD, NTD>(oacc, aP, bU);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const long t = t0 + 16 * jb + 4 * g + e;
                    if (t < p.T) {
                        const long oi = (bh * p.T + t) * p.dv + col;
                        if (p.o_bf16)
                            static_cast<uint16_t*>(p.o)[oi] = f32_to_bf16_bits(oacc[e]);
                        else
                            static_cast<float*>(p.o)[oi] = oacc[e];
                    }
                }
                // S <- Diag(Gamma_15) S + Khat^T U
                bf16x4 bUs[NTD];
                if constexpr (VEC) {
#pragma unroll
                    for (int t2 = 0; t2 < NTD; ++t2) bUs[t2] = bU[t2];
                } else {
                    const float* sc = reinterpret_cast<const float*>(smem + C::F_SC);
                    float us[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) us[e] = uv[e] * sc[4 * CH + 16 * jb + 4 * g + e];
                    split4<NTD>(us, bUs);
                }
#pragma unroll
                for (int ib = 0; ib < NIB; ++ib) {
                    if constexpr (VEC) {
                        const float* gC = reinterpret_cast<const float*>(smem + C::V_GC);
                        const float* sE = reinterpret_cast<const float*>(smem + C::V_E);
#pragma unroll
                        for (int e = 0; e < 4; ++e) sacc[ib][e] *= gC[jb * DK + 16 * ib + 4 * g + e];
                        bf16x4 aE[NTD];
                        f32_op4<NTD>(sE + (16 * ib + ln) * C::ES + 16 * jb + 4 * g, aE);
                        mma16<NTD, NTD>(sacc[ib], aE, bUs);
                    } else {
                        const float gcs = reinterpret_cast<const float*>(smem + C::F_SC)[6 * CH + jb];
                        const RawT* sKT = reinterpret_cast<const RawT*>(smem + C::F_KT);
                        sacc[ib] *= gcs;
                        bf16x4 aE[NTR];
                        raw_op4<F32IN>(sKT + (16 * ib + ln) * C::CT + 16 * jb + 4 * g, aE);
                        mma16<NTR, NTD>(sacc[ib], aE, bUs);
                    }
                }
            }
        }
    }

    if (p.ST) {
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.ST[(bh * DK + 16 * ib + 4 * g + e) * p.dv + col] = sacc[ib][e];
    }
    if constexpr (VEC) {
        if (p.AT && tile == 0) {
            __syncthreads();
            const float* Ac = reinterpret_cast<const float*>(smem + C::V_AC);
            for (int pc = tid; pc < DK; pc += C::NTHR) p.AT[bh * DK + unperm_col(pc)] = Ac[pc];
        }
    }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------

template <int DK, int NW, bool F32IN, bool VEC>
hipError_t launch_t(const ChunkParams& p, long nbh, hipStream_t st) {
    using C = Cfg<DK, NW, F32IN, VEC>;
    const long nblk = nbh * (p.dv / C::DVT);
    chunk_fwd_kernel<DK, NW, F32IN, VEC><<<dim3(static_cast<unsigned>(nblk)), dim3(C::NTHR), 0, st>>>(p);
    return hipGetLastError();
}

template <int DK, bool F32IN, bool VEC>
hipError_t launch_nw(const ChunkParams& p, long nbh, int nw, hipStream_t st) {
    if constexpr (VEC) {
        if (nw == 4) {
            if constexpr (!F32IN) return launch_t<DK, 4, F32IN, VEC>(p, nbh, st);
            else return launch_t<DK, 2, F32IN, VEC>(p, nbh, st);
        }
        return launch_t<DK, 2, F32IN, VEC>(p, nbh, st);
    } else {
        if (nw == 4) return launch_t<DK, 4, F32IN, VEC>(p, nbh, st);
        if (nw == 2) return launch_t<DK, 2, F32IN, VEC>(p, nbh, st);
        return launch_t<DK, 1, F32IN, VEC>(p, nbh, st);
    }
}

// Waves per workgroup: the largest that still gives at least one workgroup
// per compute unit, within what the dv tiling and the gate path allow.
int choose_nw(long nbh, int dv, bool vec, bool f32in, int ncu) {
    const int cands[3] = {4, 2, 1};
    int best = 0;
    for (int nw : cands) {
        if (dv % (16 * nw) != 0) continue;
        if (vec && nw == 1) continue;
        if (vec && f32in && nw == 4) continue;
        if (!best) best = nw;  // largest allowed
        if (nbh * (dv / (16 * nw)) >= ncu) return nw;
        best = nw;             // keep shrinking toward more workgroups
    }
    return best;
}

}  // namespace

size_t chunk_fwd_workspace_bytes(const pdn_chunk_fwd_args& a) {
    if (a.T <= 0) return 0;
    if (chunk_fact_supported(a)) return chunk_fact_workspace_bytes(a);
    if (chunk_vec_supported(a)) return chunk_vec_workspace_bytes(a);
    return 0;
}

hipError_t launch_chunk_fwd(const pdn_chunk_fwd_args& a, hipStream_t stream) {
    if (a.T > 0 && chunk_fact_supported(a)) return launch_chunk_fact(a, stream);
    if (a.T > 0 && chunk_vec_supported(a)) return launch_chunk_vec(a, stream);
    ChunkParams p;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.log_alpha = a.log_alpha; p.beta = a.beta;
    p.A0 = a.precond_A0; p.AT = a.precond_AT; p.S0 = a.S0; p.ST = a.ST;
    p.o = a.o;
    p.T = a.T;
    p.dv = a.dv;
    p.alpha_mode = a.alpha_mode; p.beta_mode = a.beta_mode;
    if (a.gamma_mode == PDN_GATE_VEC) {
        p.gsrc = a.gamma; p.gts = a.dv; p.gvec = 1;
    } else if (a.gamma_mode == PDN_GATE_SCALAR) {
        p.gsrc = a.gamma; p.gts = 1; p.gvec = 0;
    } else if (a.beta_mode == PDN_GATE_VEC) {  // same as beta (dk == dv)
        p.gsrc = a.beta; p.gts = a.dk; p.gvec = 1;
    } else {
        p.gsrc = a.beta; p.gts = 1; p.gvec = 0;
    }
    p.eps = a.precond_eps;
    p.o_bf16 = a.o_dtype == PDN_BF16;
    const bool vec = a.alpha_mode == PDN_ALPHA_VEC || a.beta_mode == PDN_GATE_VEC ||
                     a.precond_eps >= 0.0f;
    const bool f32in = a.qkv_dtype == PDN_F32;
    const long nbh = static_cast<long>(a.B) * a.H;
    const int nw = choose_nw(nbh, a.dv, vec, f32in, device_cu_count());
    if (nw == 0) return hipErrorNotSupported;
    if (a.dk == 128) {
        if (vec) return f32in ? launch_nw<128, true, true>(p, nbh, nw, stream)
                              : launch_nw<128, false, true>(p, nbh, nw, stream);
        return f32in ? launch_nw<128, true, false>(p, nbh, nw, stream)
                     : launch_nw<128, false, false>(p, nbh, nw, stream);
    }
    if (vec) return f32in ? launch_nw<64, true, true>(p, nbh, nw, stream)
                          : launch_nw<64, false, true>(p, nbh, nw, stream);
    return f32in ? launch_nw<64, true, false>(p, nbh, nw, stream)
                 : launch_nw<64, false, false>(p, nbh, nw, stream);
}

}  // namespace pdn
