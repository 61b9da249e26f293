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
//   waves 2-3 ("helpers"): while the chain waves work on chunk c, they load
//     chunk c+1 from HBM and build everything the chain needs for it: the key
//     and query tiles (XOR-swizzled bf16), the gate-scaled value tile, the
//     per-token row scales, P, and M (helper 2 forms T^T with MFMAs, inverts
//     the 16x16 diagonal blocks by forward substitution and fills the
//     off-diagonal blocks with MFMAs; helper 3 forms P and stages q, v).
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
constexpr int VS = DVT + 4;  // fp32 value tile row stride

// LDS layout (bytes).  Per buffer: K, Q (bf16 [64][128], swizzled), M, P
// (fp32 [64][64], k-permuted columns, swizzled), V (fp32 [64][VS]), scalars.
constexpr int B_K = 0;
constexpr int B_Q = B_K + CH * DK * 2;
constexpr int B_M = B_Q + CH * DK * 2;
constexpr int B_P = B_M + CH * CH * 4;
constexpr int B_V = B_P + CH * CH * 4;
constexpr int B_SC = B_V + CH * VS * 4;
constexpr int SC_FLOATS = 3 * CH + 4;  // rsKS[64], rq[64], rk[64], gC
constexpr int BUF = B_SC + ((SC_FLOATS * 4 + 15) / 16) * 16;
constexpr int SCR = 2 * BUF;           // helper-2 scratch: 4 diagonal 16x16 blocks
constexpr int SCR_STRIDE = 16 * 20 + 16;  // floats between blocks
constexpr int LDS_BYTES = SCR + 4 * SCR_STRIDE * 4;
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

// M/P tiles: element (row r, physical column pc) of a [64][64] fp32 tile with
// the 16-byte chunks XORed with r % 16.
__device__ __forceinline__ int mp_off(int r, int pc) {
    return r * CH + ((((pc >> 2) ^ (r & 15)) << 2) | (pc & 3));
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

// ---------------------------------------------------------------------------
// helper-wave pieces
// ---------------------------------------------------------------------------

// Rows of a chunk in MFMA operand layout: lane (ln, g) holds, for row block
// R and k-step t, the 8 channels 32t + 8g .. +7 of token 16R + ln.
struct RowOps {
    uint4 d[4][4];  // [R][t]
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

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

// Per-token gate quantities of one chunk, one token per lane (lane < 64):
// inclusive cumulative log2 decay G2 and sqrt(beta); rows past T get G2 held
// and sb = 0 (no erase, no write).
struct Gates {
    float G2, sb, G2last;
};

__device__ __forceinline__ Gates chunk_gates(const FactParams& p, long bh, long t0, int lane,
                                             float la_raw, float be_raw) {
    const bool ok = t0 + lane < p.T;
    float gl = (p.has_alpha && ok) ? fmaxf(la_raw, kLogAlphaMin) * kLog2e : 0.0f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(gl, d, 64);
        if (lane >= d) gl += o;
    }
    Gates G;
    G.G2 = gl;
    G.sb = ok ? sqrtf(be_raw) : 0.0f;
    G.G2last = __shfl(gl, 63, 64);
    return G;
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
    const bool chain = wave < NCHAIN;

    // ---------------- helper state ----------------
    RowOps kops, qops;          // current chunk's rows (helpers)
    float la_raw = 0.f, be_raw = 0.f;
    uint4 vraw[4];              // helper 3: value tile pieces (row, 8 columns)
    f32x4 gam[8];               // helper 3: value gains (per column) ...
    float gam1[4];              // ... or one per row
    auto issue_loads = [&](long t0) {
        const long tok = bh * p.T + min(t0 + lane, p.T - 1);
        la_raw = p.log_alpha[tok];
        be_raw = p.beta[tok];
        load_rows(kops, p.k, bh, p.T, t0, ln, g);
        if (wave == NCHAIN + 1) {
            load_rows(qops, p.q, bh, p.T, t0, ln, g);
#pragma unroll
            for (int m = 0; m < 4; ++m) {  // 64 rows x 4 pieces of 8 columns
                const int pi = lane + 64 * m;
                const int row = pi >> 2, c0 = (pi & 3) * 8;
                const long tk = bh * p.T + min(t0 + row, p.T - 1);
                vraw[m] = *reinterpret_cast<const uint4*>(p.v + tk * p.dv + j0 + c0);
                if (p.gvec) {
                    gam[2 * m] = *reinterpret_cast<const f32x4*>(p.gsrc + tk * p.gts + j0 + c0);
                    gam[2 * m + 1] = *reinterpret_cast<const f32x4*>(p.gsrc + tk * p.gts + j0 + c0 + 4);
                } else {
                    gam1[m] = p.gsrc[tk * p.gts];
                }
            }
        }
    };

    // Build everything chunk `c` needs into buffer `buf` (helper waves only).
    auto prepare = [&](long c, char* buf) {
        const long t0 = c * CH;
        mask_rows(kops, p.T, t0, ln);
        const Gates G = chunk_gates(p, bh, t0, lane, la_raw, be_raw);
        if (wave == NCHAIN) {
            // ---- helper 2: stage K, form T^T, invert, write M ----
            stage_rows(kops, reinterpret_cast<uint16_t*>(buf + B_K), ln, g);
            float* scr = reinterpret_cast<float*>(smem + SCR);
            // T^T blocks: tt[R][J] holds T[16R + ln][16J + 4g + e] (J < R) in registers;
            // diagonal blocks go to the scratch in natural layout.
            f32x4 tt[4][4];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int J = 0; J <= R; ++J) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        acc = mfma32(as_bf16x8(kops.d[J][t]), as_bf16x8(kops.d[R][t]), acc);
                    const int r = 16 * R + ln;
                    const float G2r = __shfl(G.G2, r, 64), sbr = __shfl(G.sb, r, 64);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * J + 4 * g + e;
                        const float G2s = __shfl(G.G2, s, 64), sbs = __shfl(G.sb, s, 64);
                        acc[e] = (s < r) ? acc[e] * sbr * sbs * exp2f(G2r - G2s) : 0.0f;
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
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = (r == cc) ? 1.0f : 0.0f;
#pragma unroll
                for (int r = 1; r < 16; ++r) {
                    float acc = 0.0f;
#pragma unroll
                    for (int j = 0; j < r; ++j) acc = fmaf(B[r * 20 + j], x[j], acc);
                    if (r > cc) x[r] = -acc;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) B[r * 20 + cc] = x[r];
            }
            // D_S in accumulator layout (lane holds D_S[4g+e][ln]) and -D_R as A operand
            auto dblk = [&](int S) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = scr[S * SCR_STRIDE + (4 * g + e) * 20 + ln];
                return v;
            };
            auto negd_a = [&](int R, bf16x4 (&a)[2]) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(scr + R * SCR_STRIDE + ln * 20 + 4 * g);
                float x[4] = {-v[0], -v[1], -v[2], -v[3]};
                split4<2>(x, a);
            };
            // M_RS = -D_R sum_{J=S}^{R-1} T_RJ M_JS, in accumulator layout.
            // T_RJ M_JS = X^T Y with X = T_RJ^T (held) and Y = M_JS (held).
            f32x4 mo[4][4];
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
                        split_d(J == S ? dblk(S) : mo[J][S], b);
                        w = mm22x16(a, b, w);
                    }
                    bf16x4 a[2], b[2];
                    negd_a(R, a);
                    split_d(w, b);
                    f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    mo[R][S] = mm22x16(a, b, z);
                }
            // write M (fp32, k-permuted swizzled); zero the upper blocks the chain reads
            float* sM = reinterpret_cast<float*>(buf + B_M);
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int S = 0; S < 4; ++S) {
                    if (S > R && !((R == 0 && S == 1) || (R == 2 && S == 3))) continue;
                    f32x4 v = {0.f, 0.f, 0.f, 0.f};
                    if (S == R) v = dblk(R);
                    else if (S < R) v = mo[R][S];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sM[mp_off(16 * R + 4 * g + e, kperm(16 * S + ln))] = v[e];
                }
        } else {
            // ---- helper 3: stage Q, V, scalars; form P ----
            mask_rows(qops, p.T, t0, ln);
            stage_rows(qops, reinterpret_cast<uint16_t*>(buf + B_Q), ln, g);
            float* sc = reinterpret_cast<float*>(buf + B_SC);
            sc[lane] = G.sb * exp2f(G.G2);                    // rows of K.Gamma
            sc[CH + lane] = exp2f(G.G2);                      // rows of Q.Gamma
            sc[2 * CH + lane] = G.sb * exp2f(G.G2last - G.G2);  // rows of Khat
            if (lane == 0) sc[3 * CH] = exp2f(G.G2last);       // chunk decay
            float* sV = reinterpret_cast<float*>(buf + B_V);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int pi = lane + 64 * m;
                const int row = pi >> 2, c0 = (pi & 3) * 8;
                const bool ok = t0 + row < p.T;
                const uint16_t* ve = reinterpret_cast<const uint16_t*>(&vraw[m]);
                f32x4 o0, o1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float g0 = p.gvec ? gam[2 * m][e] : gam1[m];
                    const float g1 = p.gvec ? gam[2 * m + 1][e] : gam1[m];
                    o0[e] = ok ? sqrtf(g0) * bf16_bits_to_f32(ve[e]) : 0.0f;
                    o1[e] = ok ? sqrtf(g1) * bf16_bits_to_f32(ve[4 + e]) : 0.0f;
                }
                *reinterpret_cast<f32x4*>(sV + row * VS + c0) = o0;
                *reinterpret_cast<f32x4*>(sV + row * VS + c0 + 4) = o1;
            }
            float* sP = reinterpret_cast<float*>(buf + B_P);
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int S = 0; S < 4; ++S) {
                    if (S > R && !((R == 0 && S == 1) || (R == 2 && S == 3))) continue;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if (S <= R) {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            acc = mfma32(as_bf16x8(qops.d[R][t]), as_bf16x8(kops.d[S][t]), acc);
                        const int s = 16 * S + ln;
                        const float G2s = __shfl(G.G2, s, 64), sbs = __shfl(G.sb, s, 64);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 16 * R + 4 * g + e;
                            const float G2r = __shfl(G.G2, r, 64);
                            acc[e] = (s <= r) ? acc[e] * sbs * exp2f(G2r - G2s) : 0.0f;
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sP[mp_off(16 * R + 4 * g + e, kperm(16 * S + ln))] = acc[e];
                }
        }
    };

    // The two roles run separate loops with the same number of barriers, so
    // their register live ranges do not overlap.
    if (chain) {
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
            const float* sM = reinterpret_cast<const float*>(cur + B_M);
            const float* sP = reinterpret_cast<const float*>(cur + B_P);
            const float* sV = reinterpret_cast<const float*>(cur + B_V);
            const float* sc = reinterpret_cast<const float*>(cur + B_SC);
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
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * a + 4 * g + e;
                    x[a][e] = sV[r * VS + 16 * wave + ln] - sc[r] * y[a][e];
                }
            bf16x8 bX[2][2];
            split_pair(x[0], x[1], bX[0]);
            split_pair(x[2], x[3], bX[1]);
            // U = M X  (M lower triangular: block row R uses k-steps t <= R/2)
            f32x4 u[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                u[R] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t <= R / 2; ++t) {
                    float mv[8];
                    const int r = 16 * R + ln, pc = 32 * t + 8 * g;
                    *reinterpret_cast<f32x4*>(mv) = *reinterpret_cast<const f32x4*>(sM + mp_off(r, pc));
                    *reinterpret_cast<f32x4*>(mv + 4) = *reinterpret_cast<const f32x4*>(sM + mp_off(r, pc + 4));
                    bf16x8 am[2];
                    split8<2>(mv, am);
                    u[R] = mm22(am, bX[t], u[R]);
                }
            }
            bf16x8 bU[2][2];
            split_pair(u[0], u[1], bU[0]);
            split_pair(u[2], u[3], bU[1]);
            // O = diag(Gamma) Z + P U
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                f32x4 oacc;
#pragma unroll
                for (int e = 0; e < 4; ++e) oacc[e] = z[R][e] * sc[CH + 16 * R + 4 * g + e];
#pragma unroll
                for (int t = 0; t <= R / 2; ++t) {
                    float pv[8];
                    const int r = 16 * R + ln, pc = 32 * t + 8 * g;
                    *reinterpret_cast<f32x4*>(pv) = *reinterpret_cast<const f32x4*>(sP + mp_off(r, pc));
                    *reinterpret_cast<f32x4*>(pv + 4) = *reinterpret_cast<const f32x4*>(sP + mp_off(r, pc + 4));
                    bf16x8 ap[2];
                    split8<2>(pv, ap);
                    oacc = mm22(ap, bU[t], oacc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const long t = t0 + 16 * R + 4 * g + e;
                    if (t < p.T) {
                        const long oi = (bh * p.T + t) * p.dv + col;
                        if (p.o_bf16) static_cast<uint16_t*>(p.o)[oi] = f32_to_bf16_bits(oacc[e]);
                        else static_cast<float*>(p.o)[oi] = oacc[e];
                    }
                }
            }
            // S <- Gamma_63 S + K^T diag(sb exp(G_63 - G)) U
            f32x4 us[4];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int e = 0; e < 4; ++e) us[R][e] = u[R][e] * sc[2 * CH + 16 * R + 4 * g + e];
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
                    const int q4 = ln & 3, jj = ln >> 2;
                    const int pcol = kperm(16 * ib + 4 * q4);
                    const int tokA = 32 * t + 4 * g + jj, tokB = tokA + 16;
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(sK + kq_off(tokA, pcol)));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(sK + kq_off(tokB, pcol)));
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
    } else {
        if (nchunks > 0) {
            issue_loads(0);
            prepare(0, smem);
            if (nchunks > 1) issue_loads(CH);
        }
        __syncthreads();
        for (long c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) {
                prepare(c + 1, smem + ((c + 1) & 1) * BUF);
                if (c + 2 < nchunks) issue_loads((c + 2) * CH);
            }
            __syncthreads();
        }
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
    p.log_alpha = p.has_alpha ? a.log_alpha : a.beta;  // never read when no decay
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
