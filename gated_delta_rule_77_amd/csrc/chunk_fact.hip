// Prefill for per-token scalar decay and gain (Gated DeltaNet / DeltaNet
// gating), bf16 q/k/v, dk = 128: the throughput path.
//
// Same chunk algebra as chunk_fwd.hip, but over whole 64-token chunks with a
// precomputed 64x64 (I+T)^-1 ("Gated DeltaNet-2" method section 3: decay
// absorbed into the erase/write matrices, one unit-lower-triangular solve per
// chunk).  With G_r the cumulative log decay from the chunk start,
// Gamma_r = exp(G_r), sb_r = sqrt(beta_r):
//
//   T_rs = sb_r sb_s exp(G_r - G_s) (k_r . k_s)      s < r
//   P_rs = sb_s exp(G_r - G_s) (q_r . k_s)           s <= r
//   M    = (I + T)^-1
//   U    = M (Vt - diag(sb Gamma) K S)
//   O    = diag(Gamma) Q S + P U
//   S   <- Gamma_63 S + K^T diag(sb exp(G_63 - G)) U
//
// Work split.  A workgroup owns (b, h, 32 value columns) for the whole
// sequence and has four waves:
//   waves 0-1 ("chain"): 16 state columns each, held in MFMA accumulator
//     registers; per chunk 132 bf16 MFMAs (16x16x32) on hi/lo-split operands.
//   waves 2-3 ("helpers"): while the chain waves work on chunk c, they build
//     everything chunk c+1 needs, from data they loaded two chunks ahead:
//     wave 2 stages the key tile, forms T with MFMAs, inverts its 16x16
//     diagonal blocks by forward substitution and fills the off-diagonal
//     blocks of M with MFMAs; wave 3 stages the query tile, the gate-scaled
//     value tile and the per-row scales, and forms P.  M and P are written
//     already split into bf16 hi/lo fragments in the per-lane order of the
//     chain's MFMA operands, so the chain reads them with one 16-byte load
//     per term and no conversion.
// LDS holds two chunk buffers; one workgroup barrier per chunk hands a
// buffer from the helpers to the chain waves.  The state-update operand K^T
// is read from the row-major key tile with the gfx950 LDS transpose read
// (ds_read_b64_tr_b16), so no transposed copy of K is stored.
#include "common.h"
#include "kernels.h"

namespace pdn {
namespace {

constexpr int DK = 128;
constexpr int CH = 64;
constexpr int NCHAIN = 2;
constexpr int NTHR = 64 * (NCHAIN + 2);
constexpr int DVT = 16 * NCHAIN;
constexpr int VTS = CH + 4;  // row stride of the transposed value tile (floats)
constexpr int NFRAG = 6;     // lower-triangular (block row, k-step) operand fragments

// LDS layout (bytes).  Per buffer: K, Q (bf16 [64][128], swizzled), M and P
// fragments, the value tile transposed (fp32 [32][VTS]), per-row scales.
constexpr int B_K = 0;
constexpr int B_Q = B_K + CH * DK * 2;
constexpr int B_MF = B_Q + CH * DK * 2;
constexpr int B_PF = B_MF + NFRAG * 2 * 64 * 16;
constexpr int B_VT = B_PF + NFRAG * 2 * 64 * 16;
constexpr int B_SC = B_VT + DVT * VTS * 4;
constexpr int BUF = B_SC + 4 * CH * 4;  // rsKS[64], rq[64], rk[64], gC
constexpr int SCR = 2 * BUF;            // wave 2: four diagonal 16x16 blocks
constexpr int SCR_STRIDE = 16 * 20 + 16;
constexpr int GA = SCR + 4 * SCR_STRIDE * 4;  // per helper: G2[64], sb[64]
constexpr int LDS_BYTES = GA + 2 * 2 * CH * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

struct FactParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* log_alpha;  // may alias beta when there is no decay
    const float* beta;
    const float* gsrc;
    long gts;
    const float* S0;
    float* ST;
    void* o;
    long T;
    int dv;
    int has_alpha;
    int gvec;
    int o_bf16;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---------------------------------------------------------------------------
// layouts
// ---------------------------------------------------------------------------

// k-permutation inside each 32-column group (see chunk_fwd.hip): one 16-byte
// read yields the k-slots {4g..4g+3, 16+4g..16+4g+3}.
__device__ __forceinline__ int kperm(int k) {
    const int q = k >> 2;
    const int pq = (q & ~7) | ((q & 3) << 1) | ((q >> 2) & 1);
    return (pq << 2) | (k & 3);
}

// K/Q tiles: element (token r, physical column pc) of a [64][128] bf16 tile.
// 16-byte chunks are XORed with f(r) = 4 (r % 4) + (r / 4) % 4, which makes
// both the 16-row MFMA operand reads and the 4x4 transpose reads hit 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int kq_off(int r, int pc) {
    const int f = ((r & 3) << 2) | ((r >> 2) & 3);
    return r * DK + ((((pc >> 3) ^ f) << 3) | (pc & 7));
}

// Byte offset of term `plane` (0 = hi, 1 = lo) for `lane` in the fragment of
// (block row R, k-step t), t <= R / 2.
__device__ __forceinline__ int frag_off(int R, int t, int plane, int lane) {
    const int f = (R < 2) ? R : 2 + 2 * (R - 2) + t;
    return ((f * 2 + plane) * 64 + lane) * 16;
}

template <int NT>
__device__ __forceinline__ void split8(const float* x, bf16x8 (&o)[NT]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
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
__device__ __forceinline__ void split4(const float* x, bf16x4 (&o)[NT]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float r = x[e];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bf16 h = static_cast<bf16>(r);
            o[t][e] = h;
            if (t + 1 < NT) r -= static_cast<float>(h);
        }
    }
}

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// acc += a (1 term) * b (hi, lo)
__device__ __forceinline__ f32x4 mm12(const bf16x8& a, const bf16x8 (&b)[2], f32x4 c) {
    c = mfma32(a, b[1], c);
    return mfma32(a, b[0], c);
}
// acc += (hi, lo) * (hi, lo), dropping lo*lo
__device__ __forceinline__ f32x4 mm22(const bf16x8 (&a)[2], const bf16x8 (&b)[2], f32x4 c) {
    c = mfma32(a[1], b[0], c);
    c = mfma32(a[0], b[1], c);
    return mfma32(a[0], b[0], c);
}
__device__ __forceinline__ f32x4 mm22x16(const bf16x4 (&a)[2], const bf16x4 (&b)[2], f32x4 c) {
    c = mfma16(a[1], b[0], c);
    c = mfma16(a[0], b[1], c);
    return mfma16(a[0], b[0], c);
}

__device__ __forceinline__ void split_d(const f32x4& v, bf16x4 (&o)[2]) {
    float x[4] = {v[0], v[1], v[2], v[3]};
    split4<2>(x, o);
}
__device__ __forceinline__ void split_pair(const f32x4& lo4, const f32x4& hi4, bf16x8 (&o)[2]) {
    float x[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    split8<2>(x, o);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

// ---------------------------------------------------------------------------
// helper-wave pieces
// ---------------------------------------------------------------------------

// Rows of a chunk in MFMA operand layout: lane (ln, g) holds, for row block
// R and k-step t, the 8 channels 32t + 8g .. +7 of token 16R + ln.
struct RowOps {
    uint4 d[4][4];  // [R][t]
};

// One chunk's raw inputs as loaded by a helper wave.
struct HelperRegs {
    RowOps k, q;    // q: wave 3 only
    uint4 v[4];     // wave 3: this lane's token, value columns 8m .. 8m + 7
    float gam1;     // wave 3: this lane's scalar value gain
    float la, be;   // this lane's token
};

__device__ __forceinline__ void load_rows(RowOps& ops, const uint16_t* base, long bh, long T,
                                          long t0, int ln, int g) {
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        const long t = min(t0 + 16 * R + ln, T - 1);
        const uint16_t* row = base + (bh * T + t) * DK;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) ops.d[R][tt] = *reinterpret_cast<const uint4*>(row + 32 * tt + 8 * g);
    }
}

__device__ __forceinline__ void mask_rows(RowOps& ops, long T, long t0, int ln) {
#pragma unroll
    for (int R = 0; R < 4; ++R)
        if (t0 + 16 * R + ln >= T)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) ops.d[R][tt] = uint4{0u, 0u, 0u, 0u};
}

// Stage operand rows into a swizzled, k-permuted LDS tile.
__device__ __forceinline__ void stage_rows(const RowOps& ops, uint16_t* tile, int ln, int g) {
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int r = 16 * R + ln;
            const int c0 = 32 * tt + 8 * g;  // logical channels c0..c0+7 = two 4-groups
            const uint4 d = ops.d[R][tt];
            *reinterpret_cast<uint2*>(tile + kq_off(r, kperm(c0))) = uint2{d.x, d.y};
            *reinterpret_cast<uint2*>(tile + kq_off(r, kperm(c0 + 4))) = uint2{d.z, d.w};
        }
}

// Write one operand fragment (8 values of this lane) as hi/lo bf16 terms.
__device__ __forceinline__ void put_frag(char* base, int R, int t, int lane, const f32x4& lo4,
                                         const f32x4& hi4) {
    bf16x8 h[2];
    split_pair(lo4, hi4, h);
    *reinterpret_cast<bf16x8*>(base + frag_off(R, t, 0, lane)) = h[0];
    *reinterpret_cast<bf16x8*>(base + frag_off(R, t, 1, lane)) = h[1];
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(NTHR) chunk_fact_kernel(FactParams p) {
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int ln = lane & 15;
    const int ntile = p.dv / DVT;
    const long bh = blockIdx.x / ntile;
    const int j0 = (blockIdx.x % ntile) * DVT;
    const long nchunks = (p.T + CH - 1) / CH;

    if (wave < NCHAIN) {
        // =========================== chain waves ===========================
        f32x4 sacc[8];
        const int col = j0 + 16 * wave + ln;
        if (p.S0) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sacc[ib][e] = p.S0[(bh * DK + 16 * ib + 4 * g + e) * p.dv + col];
        } else {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) sacc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        for (long c = 0; c < nchunks; ++c) {
            const char* cur = smem + (c & 1) * BUF;
            const uint16_t* sK = reinterpret_cast<const uint16_t*>(cur + B_K);
            const uint16_t* sQ = reinterpret_cast<const uint16_t*>(cur + B_Q);
            const float* sc = reinterpret_cast<const float*>(cur + B_SC);
            const float* sVt = reinterpret_cast<const float*>(cur + B_VT) + (16 * wave + ln) * VTS;
            const long t0 = c * CH;

            // state as x32 B operands (k = key channel)
            bf16x8 bS[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) split_pair(sacc[2 * t], sacc[2 * t + 1], bS[t]);
            // Y = K S, Z = Q S (raw bf16 rows as A operands)
            f32x4 y[4], z[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                y[a] = f32x4{0.f, 0.f, 0.f, 0.f};
                z[a] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int r = 16 * a + ln;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int pc = 32 * t + 8 * g;
                    const bf16x8 ak = *reinterpret_cast<const bf16x8*>(sK + kq_off(r, pc));
                    const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQ + kq_off(r, pc));
                    y[a] = mm12(ak, bS[t], y[a]);
                    z[a] = mm12(aq, bS[t], z[a]);
                }
            }
            // X = Vt - diag(sb Gamma) Y
            f32x4 x[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 rs = *reinterpret_cast<const f32x4*>(sc + 16 * a + 4 * g);
                const f32x4 vv = *reinterpret_cast<const f32x4*>(sVt + 16 * a + 4 * g);
                x[a] = vv - rs * y[a];
            }
            bf16x8 bX[2][2];
            split_pair(x[0], x[1], bX[0]);
            split_pair(x[2], x[3], bX[1]);
            // U = M X  (M lower triangular: block row R uses k-steps t <= R/2)
            const char* mf = cur + B_MF;
            f32x4 u[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                u[R] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t <= R / 2; ++t) {
                    bf16x8 am[2];
                    am[0] = *reinterpret_cast<const bf16x8*>(mf + frag_off(R, t, 0, lane));
                    am[1] = *reinterpret_cast<const bf16x8*>(mf + frag_off(R, t, 1, lane));
                    u[R] = mm22(am, bX[t], u[R]);
                }
            }
            bf16x8 bU[2][2];
            split_pair(u[0], u[1], bU[0]);
            split_pair(u[2], u[3], bU[1]);
            // O = diag(Gamma) Z + P U
            const char* pf = cur + B_PF;
            const bool full = t0 + CH <= p.T;
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const f32x4 rq = *reinterpret_cast<const f32x4*>(sc + CH + 16 * R + 4 * g);
                f32x4 oacc = rq * z[R];
#pragma unroll
                for (int t = 0; t <= R / 2; ++t) {
                    bf16x8 ap[2];
                    ap[0] = *reinterpret_cast<const bf16x8*>(pf + frag_off(R, t, 0, lane));
                    ap[1] = *reinterpret_cast<const bf16x8*>(pf + frag_off(R, t, 1, lane));
                    oacc = mm22(ap, bU[t], oacc);
                }
                const long row0 = (bh * p.T + t0 + 16 * R + 4 * g) * p.dv + col;
                if (p.o_bf16) {
                    uint16_t* op = static_cast<uint16_t*>(p.o) + row0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (full || t0 + 16 * R + 4 * g + e < p.T) op[e * p.dv] = f32_to_bf16_bits(oacc[e]);
                } else {
                    float* op = static_cast<float*>(p.o) + row0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (full || t0 + 16 * R + 4 * g + e < p.T) op[e * p.dv] = oacc[e];
                }
            }
            // S <- Gamma_63 S + K^T diag(sb exp(G_63 - G)) U
            f32x4 us[4];
#pragma unroll
            for (int R = 0; R < 4; ++R)
                us[R] = u[R] * *reinterpret_cast<const f32x4*>(sc + 2 * CH + 16 * R + 4 * g);
            bf16x8 bUs[2][2];
            split_pair(us[0], us[1], bUs[0]);
            split_pair(us[2], us[3], bUs[1]);
            const float gC = sc[3 * CH];
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) {
                sacc[ib] *= gC;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    // A operand: K^T rows 16ib..16ib+15 (channels), k-slots = tokens
                    // {32t + 4g + 0..3, 32t + 16 + 4g + 0..3}, via transpose reads.
                    const int pcol = kperm(16 * ib + 4 * (ln & 3));
                    const int tokA = 32 * t + 4 * g + (ln >> 2);
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(sK + kq_off(tokA, pcol)));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(sK + kq_off(tokA + 16, pcol)));
                    // whole-vector reinterpretation (an element-wise short -> bf16
                    // bit_cast loop is mis-lowered by this compiler: it replicates
                    // element 0)
                    const bf16x8 ak = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    sacc[ib] = mm12(ak, bUs[t], sacc[ib]);
                }
            }
            __syncthreads();
        }
        if (p.ST) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p.ST[(bh * DK + 16 * ib + 4 * g + e) * p.dv + col] = sacc[ib][e];
        }
        return;
    }

    // ============================= helper waves =============================
    const bool w2 = wave == NCHAIN;  // else wave 3
    float* ga = reinterpret_cast<float*>(smem + GA) + (w2 ? 0 : 2 * CH);

    auto load = [&](long c, HelperRegs& H) {
        const long t0 = c * CH;
        const long tok = bh * p.T + min(t0 + lane, p.T - 1);
        H.la = p.log_alpha[tok];
        H.be = p.beta[tok];
        load_rows(H.k, p.k, bh, p.T, t0, ln, g);
        if (!w2) {
            load_rows(H.q, p.q, bh, p.T, t0, ln, g);
#pragma unroll
            for (int m = 0; m < 4; ++m) {  // this lane's token, columns 8m .. 8m + 7
                const int row = lane, c0 = 8 * m;
                const long tk = bh * p.T + min(t0 + row, p.T - 1);
                H.v[m] = *reinterpret_cast<const uint4*>(p.v + tk * p.dv + j0 + c0);
            }
            if (!p.gvec) H.gam1 = p.gsrc[tok * p.gts];
        }
    };

    // Build everything chunk c needs into `buf` from the registers in H.
    auto prepare = [&](long c, char* buf, HelperRegs& H) {
        const long t0 = c * CH;
        mask_rows(H.k, p.T, t0, ln);
        // per-token gates: inclusive cumulative log2 decay and sqrt(beta);
        // rows past T hold G and get sb = 0 (no erase, no write)
        const bool ok = t0 + lane < p.T;
        float gl = (p.has_alpha && ok) ? fmaxf(H.la, kLogAlphaMin) * kLog2e : 0.0f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float o = __shfl_up(gl, d, 64);
            if (lane >= d) gl += o;
        }
        const float sb = ok ? sqrtf(H.be) : 0.0f;
        const float G2last = __shfl(gl, 63, 64);
        ga[lane] = gl;
        ga[CH + lane] = sb;
        // gate values at rows 16R + ln and at columns 16J + 4g + e
        float Gr[4], sbr[4];
        f32x4 Gs[4], sbs[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            Gr[R] = ga[16 * R + ln];
            sbr[R] = ga[CH + 16 * R + ln];
            Gs[R] = *reinterpret_cast<const f32x4*>(ga + 16 * R + 4 * g);
            sbs[R] = *reinterpret_cast<const f32x4*>(ga + CH + 16 * R + 4 * g);
        }

        if (w2) {
            // ---- wave 2: form T, stage K, invert, write M fragments ----
            // raw key Gram blocks first, so the key registers can be refilled
            f32x4 tr[4][4];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int J = 0; J <= R; ++J) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        acc = mfma32(as_bf16x8(H.k.d[J][t]), as_bf16x8(H.k.d[R][t]), acc);
                    tr[R][J] = acc;
                }
            stage_rows(H.k, reinterpret_cast<uint16_t*>(buf + B_K), ln, g);
            if (c + 1 < nchunks) load(c + 1, H);
            float* scr = reinterpret_cast<float*>(smem + SCR);
            // tt[R][J] holds T[16R + ln][16J + 4g + e] for J < R (i.e. T_RJ^T in
            // accumulator layout); diagonal blocks go to the scratch.
            f32x4 tt[4][4];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int J = 0; J <= R; ++J) {
                    f32x4 acc = tr[R][J];
                    const int r = 16 * R + ln;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * J + 4 * g + e;
                        acc[e] = (s < r) ? acc[e] * sbr[R] * sbs[J][e] * exp2f(Gr[R] - Gs[J][e]) : 0.0f;
                    }
                    if (J == R)
                        *reinterpret_cast<f32x4*>(scr + R * SCR_STRIDE + ln * 20 + 4 * g) = acc;
                    else
                        tt[R][J] = acc;
                }
            // diagonal blocks: (I + T_RR)^-1 by forward substitution, lane = (R, column)
            {
                float* B = scr + (lane >> 4) * SCR_STRIDE;
                const int cc = lane & 15;
                float xs[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) xs[r] = (r == cc) ? 1.0f : 0.0f;
#pragma unroll
                for (int r = 1; r < 16; ++r) {
                    float acc = 0.0f;
#pragma unroll
                    for (int j = 0; j < r; ++j) acc = fmaf(B[r * 20 + j], xs[j], acc);
                    if (r > cc) xs[r] = -acc;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) B[r * 20 + cc] = xs[r];
            }
            // dcol(S): D_S[4g+e][ln] (accumulator layout); drow(R): D_R[ln][4g+e]
            auto dcol = [&](int S) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = scr[S * SCR_STRIDE + (4 * g + e) * 20 + ln];
                return v;
            };
            auto drow = [&](int R) {
                return *reinterpret_cast<const f32x4*>(scr + R * SCR_STRIDE + ln * 20 + 4 * g);
            };
            // M_RS = -D_R sum_{J=S}^{R-1} T_RJ M_JS in accumulator layout (mo), and
            // its transpose (mt) from the same operands with the roles swapped:
            // a register block used as the A operand acts as its transpose.
            f32x4 mo[4][4], mt[4][4];
#pragma unroll
            for (int d = 1; d < 4; ++d)
#pragma unroll
                for (int S = 0; S + d < 4; ++S) {
                    const int R = S + d;
                    f32x4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int J = S; J < R; ++J) {
                        bf16x4 a[2], b[2];
                        split_d(tt[R][J], a);
                        split_d(J == S ? dcol(S) : mo[J][S], b);
                        w = mm22x16(a, b, w);
                    }
                    const f32x4 dr = drow(R);
                    bf16x4 nd[2], bw[2];
                    split_d(f32x4{-dr[0], -dr[1], -dr[2], -dr[3]}, nd);
                    split_d(w, bw);
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    mo[R][S] = mm22x16(nd, bw, zero);
                    mt[R][S] = mm22x16(bw, nd, zero);
                }
            // M fragments: lane (ln, g) of fragment (R, t) holds M[16R + ln][32t + 4g + j]
            // (j < 4) and M[16R + ln][32t + 16 + 4g + j - 4]: the transposed blocks
            // (R, 2t) and (R, 2t + 1) in accumulator layout.
            char* mf = buf + B_MF;
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            put_frag(mf, 0, 0, lane, drow(0), zero);
            put_frag(mf, 1, 0, lane, mt[1][0], drow(1));
            put_frag(mf, 2, 0, lane, mt[2][0], mt[2][1]);
            put_frag(mf, 2, 1, lane, drow(2), zero);
            put_frag(mf, 3, 0, lane, mt[3][0], mt[3][1]);
            put_frag(mf, 3, 1, lane, mt[3][2], drow(3));
        } else {
            // ---- wave 3: form P, stage Q, V (transposed), row scales ----
            mask_rows(H.q, p.T, t0, ln);
            // raw query-key products first, so the registers can be refilled
            f32x4 pb[4][4];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int S = 0; S <= R; ++S) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        acc = mfma32(as_bf16x8(H.k.d[S][t]), as_bf16x8(H.q.d[R][t]), acc);
                    pb[R][S] = acc;
                }
            stage_rows(H.q, reinterpret_cast<uint16_t*>(buf + B_Q), ln, g);
            float* sc = reinterpret_cast<float*>(buf + B_SC);
            sc[lane] = sb * exp2f(gl);                    // rows of K.Gamma
            sc[CH + lane] = exp2f(gl);                    // rows of Q.Gamma
            sc[2 * CH + lane] = sb * exp2f(G2last - gl);  // rows of Khat
            if (lane == 0) sc[3 * CH] = exp2f(G2last);    // chunk decay
            float* sVt = reinterpret_cast<float*>(buf + B_VT);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int row = lane, c0 = 8 * m;
                const bool okr = t0 + row < p.T;
                const uint16_t* ve = reinterpret_cast<const uint16_t*>(&H.v[m]);
                float gam[8];
                if (p.gvec) {
                    const long tk = bh * p.T + min(t0 + row, p.T - 1);
#pragma unroll
                    for (int e = 0; e < 8; ++e) gam[e] = p.gsrc[tk * p.gts + j0 + c0 + e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) gam[e] = H.gam1;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sVt[(c0 + e) * VTS + row] = okr ? sqrtf(gam[e]) * bf16_bits_to_f32(ve[e]) : 0.0f;
            }
            if (c + 1 < nchunks) load(c + 1, H);
            // P^T blocks: pb[R][S] holds P[16R + ln][16S + 4g + e]
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int S = 0; S <= R; ++S) {
                    const int r = 16 * R + ln;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * S + 4 * g + e;
                        pb[R][S][e] = (s <= r) ? pb[R][S][e] * sbs[S][e] * exp2f(Gr[R] - Gs[S][e]) : 0.0f;
                    }
                }
            char* pf = buf + B_PF;
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            put_frag(pf, 0, 0, lane, pb[0][0], zero);
            put_frag(pf, 1, 0, lane, pb[1][0], pb[1][1]);
            put_frag(pf, 2, 0, lane, pb[2][0], pb[2][1]);
            put_frag(pf, 2, 1, lane, pb[2][2], zero);
            put_frag(pf, 3, 0, lane, pb[3][0], pb[3][1]);
            put_frag(pf, 3, 1, lane, pb[3][2], pb[3][3]);
        }
    };

    // The registers hold the inputs of the next chunk to prepare; prepare()
    // refills them with the chunk after it as soon as they have been consumed,
    // which leaves a whole chunk period for the loads to land.
    HelperRegs H;
    if (nchunks > 0) {
        load(0, H);
        prepare(0, smem, H);
    }
    __syncthreads();
    for (long c = 0; c < nchunks; ++c) {
        if (c + 1 < nchunks) prepare(c + 1, smem + ((c + 1) & 1) * BUF, H);
        __syncthreads();
    }
}

}  // namespace

bool chunk_fact_supported(const pdn_chunk_fwd_args& a) {
    return a.qkv_dtype == PDN_BF16 && a.dk == DK && a.dv % DVT == 0 &&
           a.alpha_mode != PDN_ALPHA_VEC && a.beta_mode == PDN_GATE_SCALAR &&
           a.precond_eps < 0.0f;
}

hipError_t launch_chunk_fact(const pdn_chunk_fwd_args& a, hipStream_t stream) {
    FactParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.has_alpha = a.alpha_mode != PDN_ALPHA_NONE;
    p.log_alpha = p.has_alpha ? a.log_alpha : a.beta;  // never used when there is no decay
    p.beta = a.beta;
    if (a.gamma_mode == PDN_GATE_VEC) {
        p.gsrc = a.gamma; p.gts = a.dv; p.gvec = 1;
    } else if (a.gamma_mode == PDN_GATE_SCALAR) {
        p.gsrc = a.gamma; p.gts = 1; p.gvec = 0;
    } else {
        p.gsrc = a.beta; p.gts = 1; p.gvec = 0;  // scalar beta
    }
    p.S0 = a.S0;
    p.ST = a.ST;
    p.o = a.o;
    p.T = a.T;
    p.dv = a.dv;
    p.o_bf16 = a.o_dtype == PDN_BF16;
    const long nblk = static_cast<long>(a.B) * a.H * (a.dv / DVT);
    chunk_fact_kernel<<<dim3(static_cast<unsigned>(nblk)), dim3(NTHR), 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace pdn
