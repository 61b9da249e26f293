// Prefill for per-channel decay and gains and the diagonal preconditioner
// (KDA / FG^2-GDN / Gated DeltaNet-2 gating), bf16 q/k/v, dk = 128: device
// code shared by chunk_vec.hip and chunk_vec_ilp.hip (not a public header).
//
// Chunk algebra over 32-token chunks ("Gated DeltaNet-2" method section 3:
// the cumulative decay goes into the erase/write matrices and each chunk
// solves one unit-lower-triangular system; "FG^2-GDN" 2.3: the transition is
// diagonal plus low rank).  With G_ri the cumulative log2 decay of channel i
// from the chunk start, Gamma = 2^G, and per token a read key kr_r (the one
// the state is read with), a write key kw_r (the one the correction is
// written along) and a written value vw_r:
//
//   T_rs = sum_i kr_ri kw_si 2^(G_ri - G_si)          s < r
//   P_rs = sum_i q_ri  kw_si 2^(G_ri - G_si)          s <= r
//   U    = (I + T)^-1 (Vw - (Kr . Gamma) S)
//   O    = (Q . Gamma) S + P U
//   S   <- Diag(Gamma_31) S + (Kw . 2^(G_31 - G))^T U
//
// Symmetric keys: kr = kw = sqrt(beta') (.) k, vw = sqrt(gamma) (.) v.  Erase
// gate ("Gated DeltaNet-2" method section 1): kw = k, kr = beta' (.) k,
// vw = gamma (.) v.  Write gate ("Preconditioned DeltaNet" 2.2, the gain on
// the write key): kw = beta' (.) k, kr = k, vw = v (gamma (.) v when a
// separate value gain is given).
//
// Everything that depends only on q, k and the gates is independent across
// chunks, so it runs first, fully parallel over (b, h, chunk):
//
//   vec_prep_kernel (one wave per chunk) forms the gate-scaled operands
//     Kg = Kr . Gamma, Qg = Q . Gamma, Kd = Kw . 2^(G_31 - G), the blocks of T
//     and P (fp32 MFMAs), the inverses D_R = (I + T_RR)^-1 of the two 16x16
//     diagonal blocks and N = D_1 T_10, and writes them as one chunk record
//     to the workspace: bf16 hi/lo tiles and MFMA fragments laid out exactly
//     as the chain kernel's LDS expects them.
//
//   vec_chain_kernel carries the state: one workgroup per (b, h, 32 value
//     columns); waves 0-1 hold 16 state columns each in registers and run
//     the sequential part (KS, the block solve U_0 = D_0 X_0,
//     U_1 = D_1 X_1 - N U_0, QS, PU, the state update), wave 2 copies the
//     records from HBM into LDS by DMA two chunks ahead, wave 3 stages the
//     gain-scaled value tile.  One barrier per chunk, plus an LDS flag per
//     chain wave that tells wave 2 when a buffer has been read.
//
// The per-channel decay inside a 16-token block is split around the block's
// middle token (2^(G_r - Gm) 2^(Gm - G_s)); the per-token clamp of
// log(alpha) at -10 keeps both factors below 2^116.  Between the two blocks
// the split is at the last token of block 0, where both factors are <= 1.
//
// With the preconditioner, beta'_t = beta_t / (A_t + eps) with the running
// sum A_t = A_0 + sum_{s<=t} k_s (.) k_s ("Preconditioned DeltaNet" 2.2):
// vec_ksq_kernel sums k (.) k per chunk and vec_kscan_kernel turns the sums
// into the value of A before every chunk (and A_T).  In the stabilised mode
// (Eq. 9 as read here) beta'_t = beta_t x^-(r / (1 + |r|)) with
// r = ln(A_t + eps) minus its mean over the key channels of token t; the
// preparation kernel forms the per-token means in a pass over the chunk's key
// rows before the main one.
#pragma once
#include "chunk_tile.h"
#include "kernels.h"

namespace pdn {

struct PrepParams {
    const uint16_t* q;
    const uint16_t* k;
    const float* log_alpha;  // may be null when there is no decay
    const float* beta;
    const float* astart;     // [BH][nc][DK] running k.k sum before each chunk
    char* rec;               // [BH][nc] records
    long T;
    long nc;
    long nbh;
    float eps;
    int has_alpha;
    float l2x;  // stabilised preconditioner: log2 of its bound x
};

// Launcher of the symmetric-key preparation kernel with per-channel decay and
// gain, which chunk_vec_ilp.hip builds with the instruction-level-parallelism
// scheduler (3% faster that way; with asymmetric keys or the stabilised
// preconditioner the kernel is faster with the default scheduler and is
// launched from chunk_vec.hip).
template <bool PRE>
void launch_vec_prep_sym_vec(const PrepParams& p, unsigned grid, hipStream_t s);

namespace {

using namespace tile;

constexpr int VC = 32;  // tokens per chunk
constexpr int NCHAIN = 2;
constexpr int NTHR = 64 * (NCHAIN + 2);
constexpr int DVT = 16 * NCHAIN;
constexpr int VTS = VC + 4;  // row stride of the transposed value tile (floats)

// Chunk record (bytes).  Six bf16 [32][128] tiles with the swizzle of kq_off:
// hi and lo terms of Kg, Qg, Kd.  Then the solve fragments (16x16x16 A
// operands, 8 bytes per lane and term): D_0, D_1, -N; the P fragments
// (16x16x32 B operands for row blocks 0 and 1, 16 bytes per lane and term);
// and Gamma_31 per channel (fp32).  Padded to whole KiB for the DMA.
constexpr int TILEB = VC * DK * 2;
constexpr int R_KGH = 0;
constexpr int R_KGL = TILEB;
constexpr int R_QGH = 2 * TILEB;
constexpr int R_QGL = 3 * TILEB;
constexpr int R_KDH = 4 * TILEB;
constexpr int R_KDL = 5 * TILEB;
constexpr int R_F16 = 6 * TILEB;
constexpr int R_PF = R_F16 + 3 * 2 * 64 * 8;
constexpr int R_GC = R_PF + 2 * 2 * 64 * 16;
constexpr int REC = (R_GC + DK * 4 + 1023) / 1024 * 1024;
enum { F16_D0 = 0, F16_D1 = 1, F16_N10 = 2 };

__device__ __forceinline__ int f16_off(int s, int plane, int lane) { return R_F16 + ((s * 2 + plane) * 64 + lane) * 8; }
__device__ __forceinline__ int pf_off(int R, int plane, int lane) { return R_PF + ((R * 2 + plane) * 64 + lane) * 16; }

// Chain kernel LDS.  A record goes in as two parts: part A (the Kg and Qg
// tiles) into a ring of three slots, part B (Kd, the fragments, Gamma_31) into
// one of two buffers, each followed by the value tile transposed (fp32
// [32 columns][VTS]).  With three slots, chunk c + 2's part A can be fetched
// as soon as chunk c starts (its slot was chunk c - 1's); part B waits until
// the chain waves have read chunk c's buffer.
constexpr int PA = R_KDH;       // part A: record bytes [0, PA)
constexpr int PB = REC - PA;    // part B: record bytes [PA, REC)
constexpr int B_VT = PB;        // value tile, within a part-B buffer
constexpr int BUFB = PB + DVT * VTS * 4;
constexpr int L_B = 3 * PA;     // the part-B buffers follow the three slots
constexpr int LDS_CHAIN = L_B + 2 * BUFB;
static_assert(LDS_CHAIN <= 160 * 1024, "LDS budget");
static_assert(PA % 1024 == 0 && REC % 1024 == 0 && BUFB % 16 == 0, "record alignment");

// Preparation kernel: scratch for the two diagonal blocks of each wave.
constexpr int SCR_STRIDE = 16 * 20 + 16;



// How the written value follows from v and the value gain gamma.
enum { VAL_SQRT_GAIN = 0, VAL_GAIN = 1, VAL_UNIT = 2 };

struct ChainParams {
    const uint16_t* v;
    const char* rec;
    const float* gsrc;
    long gts;
    int gvec;
    int vmode;  // VAL_*
    const float* S0;
    float* ST;
    void* o;
    long T;
    long nc;
    int dv;
    int o_bf16;
    // Sequence segments (few heads, long sequences): segment g covers chunks
    // [g cps, (g + 1) cps).  Segment 0's value columns start from S0; the
    // value columns of later segments start from 0, and those segments also
    // run DK identity-start columns (zero values) whose end state is the
    // segment's transition and whose outputs are Phi^T q per token.
    int nseg;      // 1: one pass over the whole sequence
    long cps;      // chunks per segment
    float* qh;     // [BH][T][DK] outputs of the identity columns
    float* nst;    // [BH][nseg][DK][dv] end states of the value columns
    float* phi;    // [BH][nseg][DK][DK] end states of the identity columns
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Element j (0..7) of eight packed bf16 values.
__device__ __forceinline__ float bf16_at(const uint4& u, int j) {
    const uint32_t w = j < 2 ? u.x : (j < 4 ? u.y : (j < 6 ? u.z : u.w));
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

// hi/lo split of eight values into two 16-byte words
__device__ __forceinline__ void split8(const float (&x)[8], uint4& h, uint4& l) {
    split2(x[0], x[1], h.x, l.x);
    split2(x[2], x[3], h.y, l.y);
    split2(x[4], x[5], h.z, l.z);
    split2(x[6], x[7], h.w, l.w);
}

// Stabilised preconditioner coefficient x^-(r / (1 + |r|)) of a channel with
// A + eps = aeps, r = ln(aeps) - (mean of ln over the channels); mu2 is that
// mean in log2 units and l2x = log2(x).
__device__ __forceinline__ float stab_coeff(float aeps, float mu2, float l2x) {
    const float r = (__builtin_amdgcn_logf(aeps) - mu2) * kLn2;
    return __builtin_amdgcn_exp2f(-(r / (1.0f + fabsf(r))) * l2x);
}

// Decay factors of one channel (or of a scalar decay) for the two tokens a
// lane holds: token ln of block 0 and token 16 + ln of block 1.  lg0 / lg1 are
// the clamped log2 decays of those tokens; the scans run along the 16 tokens
// of a DPP row.
struct Decay {
    float e0, ei0, e1, ei1;  // 2^(G - Gm) and 2^(Gm - G) around each block's middle token
    float f0;                // block 0: 2^(G_15 - G)
    float f1;                // block 1: 2^(G - G_15)
    float gm0, gm1;          // Gamma = 2^G
    float kd0, kd1;          // 2^(G_31 - G)
    float gc;                // 2^(G_31), the chunk decay
};

__device__ __forceinline__ Decay decay_factors(float lg0, float lg1) {
    Decay d;
    const float G0 = row_incl_scan(lg0);
    const float G15 = row_bcast<15>(G0);
    const float G1 = row_incl_scan(lg1) + G15;
    const float Gm0 = row_bcast<7>(G0);
    const float Gm1 = row_bcast<7>(G1);
    const float G31 = row_bcast<15>(G1);
    d.e0 = ex2(G0 - Gm0);
    d.ei0 = ex2(Gm0 - G0);
    d.e1 = ex2(G1 - Gm1);
    d.ei1 = ex2(Gm1 - G1);
    d.f0 = ex2(G15 - G0);
    d.f1 = ex2(G1 - G15);
    d.gm0 = ex2(G0);
    const float g15 = row_bcast<15>(d.gm0);   // 2^G_15
    const float d15 = row_bcast<15>(d.f1);    // 2^(G_31 - G_15)
    d.gm1 = d.f1 * g15;
    d.kd0 = d.f0 * d15;
    d.kd1 = ex2(G31 - G1);
    d.gc = d15 * g15;
    return d;
}

// ---------------------------------------------------------------------------
// preparation: one wave per (b, h, chunk)
// ---------------------------------------------------------------------------

// Lane (ln, g) holds tokens ln (block 0) and 16 + ln (block 1) and, in k-step
// t, the channels 32t + 8g .. 32t + 8g + 7: the MFMA operand layout, so the
// Gram blocks are formed straight from registers with 16x16x4 fp32 MFMAs
// (k-slot g of MFMA (t, j) is channel 32t + 8g + j).  Results in accumulator
// layout (lane (ln, g) holds rows 4g + e, column ln):
//   T_RR with A = Kw 2^(Gm - G) rows, B = Kr 2^(G - Gm) rows gives T_RR^T, i.e.
//     lane (ln, g) holds row ln, columns 4g + e of T_RR;
//   T_10 with A = block-1 Kr rows 2^(G - G_15), B = block-0 Kw rows 2^(G_15 - G);
//   P_RS with A = block-S write-key rows, B = block-R query rows gives P_RS^T.
// KM is the key mode (PDN_KEY_*); STAB selects the stabilised preconditioner
// coefficient (with PRE).
template <bool AVEC, bool BVEC, bool PRE, int KM, bool STAB>
__global__ void __launch_bounds__(256) vec_prep_kernel(PrepParams p) {
    __shared__ __attribute__((aligned(16))) float scr_all[4][2 * SCR_STRIDE];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int ln = lane & 15;
    const long id = blockIdx.x * 4L + wave;
    if (id >= p.nbh * p.nc) return;
    const long bh = id / p.nc;
    const long c = id % p.nc;
    char* rec = p.rec + id * REC;
    float* scr = scr_all[wave];

    long row[2];
    bool ok[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const long t = c * VC + 16 * b + ln;
        ok[b] = t < p.T;
        row[b] = bh * p.T + min(t, p.T - 1);
    }
    // per-token (scalar) gates
    float lgs[2] = {0.0f, 0.0f}, bes[2] = {0.0f, 0.0f};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (!AVEC && p.has_alpha && ok[b]) lgs[b] = fmaxf(p.log_alpha[row[b]], kLogAlphaMin) * kLog2e;
        if (!BVEC && ok[b]) bes[b] = p.beta[row[b]];
    }
    Decay ds;
    if constexpr (!AVEC) ds = decay_factors(lgs[0], lgs[1]);
    // per-token key gain: sqrt(beta') for symmetric keys, else beta' itself
    float sbs[2] = {0.0f, 0.0f};
    if constexpr (!BVEC && !PRE) {
        sbs[0] = KM == PDN_KEY_SYMMETRIC ? sqrt_hw(bes[0]) : bes[0];
        sbs[1] = KM == PDN_KEY_SYMMETRIC ? sqrt_hw(bes[1]) : bes[1];
    }

    // stabilised preconditioner: mean of log2(A + eps) over the 128 key
    // channels of each of this lane's two tokens (lanes ln, 16 + ln, 32 + ln,
    // 48 + ln hold four disjoint channel groups of the same tokens)
    float mu2[2] = {0.0f, 0.0f};
    if constexpr (PRE && STAB) {
        {
            float sl[2] = {0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int cb = 32 * t + 8 * g;
                uint4 kv[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) kv[b] = *reinterpret_cast<const uint4*>(p.k + row[b] * DK + cb);
                const float* ap = p.astart + id * DK + cb;
                const f32x4 a0v = *reinterpret_cast<const f32x4*>(ap);
                const f32x4 a1v = *reinterpret_cast<const f32x4*>(ap + 4);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float k0 = ok[0] ? bf16_at(kv[0], j) : 0.0f;
                    const float k1 = ok[1] ? bf16_at(kv[1], j) : 0.0f;
                    const float a0 = row_incl_scan(k0 * k0) + (j < 4 ? a0v[j] : a1v[j - 4]);
                    const float a1 = row_incl_scan(k1 * k1) + row_bcast<15>(a0);
                    sl[0] += __builtin_amdgcn_logf(a0 + p.eps);
                    sl[1] += __builtin_amdgcn_logf(a1 + p.eps);
                }
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                sl[b] += __shfl_xor(sl[b], 16, 64);
                sl[b] += __shfl_xor(sl[b], 32, 64);
                mu2[b] = sl[b] * (1.0f / DK);
            }
        }
    }

    f32x4 t00 = {0.f, 0.f, 0.f, 0.f}, t11 = t00, t10 = t00, p00 = t00, p11 = t00, p10 = t00;
    // k-steps in pairs (2tp, 2tp + 1): the two halves of every 128-byte line of
    // the q/k rows are loaded together, and the two halves of every record line
    // (the tile swizzle keeps them in the same pair) are stored back to back,
    // so no line is fetched twice or written back half-filled
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
    uint4 kp[2][2], qp[2][2];  // [step in pair][row block]
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            kp[u][b] = *reinterpret_cast<const uint4*>(p.k + row[b] * DK + 32 * (2 * tp + u) + 8 * g);
            qp[u][b] = *reinterpret_cast<const uint4*>(p.q + row[b] * DK + 32 * (2 * tp + u) + 8 * g);
        }
    uint4 held[2][6];  // hi/lo record words of the first step of the pair
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int t = 2 * tp + u;
        const int cb = 32 * t + 8 * g;  // this lane's first channel in k-step t
        const uint4* kr = kp[u];
        const uint4* qr = qp[u];
        float la[2][8], be[2][8], as[8];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if constexpr (AVEC) {
                const f32x4 a0 = *reinterpret_cast<const f32x4*>(p.log_alpha + row[b] * DK + cb);
                const f32x4 a1 = *reinterpret_cast<const f32x4*>(p.log_alpha + row[b] * DK + cb + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    la[b][j] = a0[j];
                    la[b][4 + j] = a1[j];
                }
            }
            if constexpr (BVEC) {
                const f32x4 b0 = *reinterpret_cast<const f32x4*>(p.beta + row[b] * DK + cb);
                const f32x4 b1 = *reinterpret_cast<const f32x4*>(p.beta + row[b] * DK + cb + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    be[b][j] = b0[j];
                    be[b][4 + j] = b1[j];
                }
            }
        }
        if constexpr (PRE) {
            const float* ap = p.astart + id * DK + cb;
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(ap);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(ap + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                as[j] = a0[j];
                as[4 + j] = a1[j];
            }
        }
        float kg[2][8], qg[2][8], kd[2][8], gcv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float k0 = ok[0] ? bf16_at(kr[0], j) : 0.0f;
            const float k1 = ok[1] ? bf16_at(kr[1], j) : 0.0f;
            const float q0 = ok[0] ? bf16_at(qr[0], j) : 0.0f;
            const float q1 = ok[1] ? bf16_at(qr[1], j) : 0.0f;
            Decay d;
            if constexpr (AVEC) {
                const float l0 = (p.has_alpha && ok[0]) ? fmaxf(la[0][j], kLogAlphaMin) * kLog2e : 0.0f;
                const float l1 = (p.has_alpha && ok[1]) ? fmaxf(la[1][j], kLogAlphaMin) * kLog2e : 0.0f;
                d = decay_factors(l0, l1);
            } else {
                d = ds;
            }
            float sb0, sb1;
            if constexpr (BVEC || PRE) {
                float b0 = BVEC ? (ok[0] ? be[0][j] : 0.0f) : bes[0];
                float b1 = BVEC ? (ok[1] ? be[1][j] : 0.0f) : bes[1];
                if constexpr (PRE) {
                    const float a0 = row_incl_scan(k0 * k0) + as[j];
                    const float a1 = row_incl_scan(k1 * k1) + row_bcast<15>(a0);
                    if constexpr (STAB) {
                        b0 *= stab_coeff(a0 + p.eps, mu2[0], p.l2x);
                        b1 *= stab_coeff(a1 + p.eps, mu2[1], p.l2x);
                    } else {
                        b0 *= __builtin_amdgcn_rcpf(a0 + p.eps);
                        b1 *= __builtin_amdgcn_rcpf(a1 + p.eps);
                    }
                }
                sb0 = KM == PDN_KEY_SYMMETRIC ? sqrt_hw(b0) : b0;
                sb1 = KM == PDN_KEY_SYMMETRIC ? sqrt_hw(b1) : b1;
            } else {
                sb0 = sbs[0];
                sb1 = sbs[1];
            }
            // read and write keys (the same value for symmetric keys)
            const float kr0 = KM == PDN_KEY_WRITE_GATE ? k0 : sb0 * k0;
            const float kr1 = KM == PDN_KEY_WRITE_GATE ? k1 : sb1 * k1;
            const float kw0 = KM == PDN_KEY_ERASE_GATE ? k0 : sb0 * k0;
            const float kw1 = KM == PDN_KEY_ERASE_GATE ? k1 : sb1 * k1;
            kg[0][j] = kr0 * d.gm0;
            kg[1][j] = kr1 * d.gm1;
            qg[0][j] = q0 * d.gm0;
            qg[1][j] = q1 * d.gm1;
            kd[0][j] = kw0 * d.kd0;
            kd[1][j] = kw1 * d.kd1;
            gcv[j] = d.gc;
            const float bd0 = kw0 * d.ei0, bd1 = kw1 * d.ei1;
            const float bo = kw0 * d.f0;
            t00 = mfma4(bd0, kr0 * d.e0, t00);
            p00 = mfma4(bd0, q0 * d.e0, p00);
            t11 = mfma4(bd1, kr1 * d.e1, t11);
            p11 = mfma4(bd1, q1 * d.e1, p11);
            t10 = mfma4(kr1 * d.f1, bo, t10);
            p10 = mfma4(bo, q1 * d.f1, p10);
        }
        // gate-scaled operand rows for the chain, hi/lo, into the swizzled tiles
        uint4 w[2][6];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            split8(kg[b], w[b][0], w[b][1]);
            split8(qg[b], w[b][2], w[b][3]);
            split8(kd[b], w[b][4], w[b][5]);
        }
        if (u == 0) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int x = 0; x < 6; ++x) held[b][x] = w[b][x];
        } else {
            constexpr int tiles[6] = {R_KGH, R_KGL, R_QGH, R_QGL, R_KDH, R_KDL};
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int off0 = 2 * kq_off(16 * b + ln, cb - 32);
                const int off1 = 2 * kq_off(16 * b + ln, cb);
#pragma unroll
                for (int x = 0; x < 6; ++x) {
                    *reinterpret_cast<uint4*>(rec + tiles[x] + off0) = held[b][x];
                    *reinterpret_cast<uint4*>(rec + tiles[x] + off1) = w[b][x];
                }
            }
        }
        if (ln == 0) {
            float* gc = reinterpret_cast<float*>(rec + R_GC) + cb;
            *reinterpret_cast<f32x4*>(gc) = f32x4{gcv[0], gcv[1], gcv[2], gcv[3]};
            *reinterpret_cast<f32x4*>(gc + 4) = f32x4{gcv[4], gcv[5], gcv[6], gcv[7]};
        }
    }
    }

    // strictly lower part of the diagonal T blocks (row ln, columns 4g + e),
    // negated as the solve consumes it, to the scratch; the upper part may hold
    // overflowed products and is dropped
#pragma unroll
    for (int R = 0; R < 2; ++R) {
        f32x4 acc = R == 0 ? t00 : t11;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = (4 * g + e < ln) ? -acc[e] : 0.0f;
        *reinterpret_cast<f32x4*>(scr + R * SCR_STRIDE + ln * 20 + 4 * g) = acc;
    }
    // D_R = (I + T_RR)^-1, one row per lane; lanes 32..63 repeat lanes 0..31
    {
        float* Brow = scr + ((lane >> 4) & 1) * SCR_STRIDE + ln * 20;
        float ntr[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(Brow + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) ntr[4 * q + e] = v[e];
        }
        float x[16];
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) x[cc] = (cc == ln) ? 1.0f : 0.0f;
        block_row_solve(x, ntr);
        if (lane < 32) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f32x4*>(Brow + 4 * q) = f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
        }
    }
    // D fragments; -N = -D_1 T_10 with the T block as the A operand (a register
    // block used as A acts as its transpose), which leaves lane (ln, g) with
    // row ln, columns 4g .. 4g + 3 of -N: its A-operand fragment
    bf16x4 bd[2][2];
#pragma unroll
    for (int R = 0; R < 2; ++R) {
        split_d(*reinterpret_cast<const f32x4*>(scr + R * SCR_STRIDE + ln * 20 + 4 * g), bd[R]);
        *reinterpret_cast<bf16x4*>(rec + f16_off(F16_D0 + R, 0, lane)) = bd[R][0];
        *reinterpret_cast<bf16x4*>(rec + f16_off(F16_D0 + R, 1, lane)) = bd[R][1];
    }
    {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        bf16x4 bt[2];
        split_d(-t10, bt);
        const f32x4 nb = mm22x16(bt, bd[1], zero);
        bf16x4 h[2];
        split_d(nb, h);
        *reinterpret_cast<bf16x4*>(rec + f16_off(F16_N10, 0, lane)) = h[0];
        *reinterpret_cast<bf16x4*>(rec + f16_off(F16_N10, 1, lane)) = h[1];
    }
    // P fragments: lane (ln, g) holds P[16R + ln][4g + e] (block 0 columns) and
    // P[16R + ln][16 + 4g + e] (block 1 columns), the 16x16x32 B operand of
    // row block R
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p00[e] = (4 * g + e <= ln) ? p00[e] : 0.0f;
            p11[e] = (4 * g + e <= ln) ? p11[e] : 0.0f;
        }
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        bf16x8 h[2];
        split_pair(p00, zero, h);
        *reinterpret_cast<bf16x8*>(rec + pf_off(0, 0, lane)) = h[0];
        *reinterpret_cast<bf16x8*>(rec + pf_off(0, 1, lane)) = h[1];
        split_pair(p10, p11, h);
        *reinterpret_cast<bf16x8*>(rec + pf_off(1, 0, lane)) = h[0];
        *reinterpret_cast<bf16x8*>(rec + pf_off(1, 1, lane)) = h[1];
    }
}

// ---------------------------------------------------------------------------
// the chain
// ---------------------------------------------------------------------------

// SEG: the segmented launch (identity-start columns, segment end states);
// a separate instantiation so that the one-pass chain carries none of it.
template <bool SEG>
__global__ void __launch_bounds__(NTHR) vec_chain_kernel(ChainParams p) {
    __shared__ __attribute__((aligned(16))) char smem[LDS_CHAIN];
    // per chain wave: the last chunk (counted from the segment start) whose
    // LDS reads have all returned; a separate LDS object, so that the
    // compiler can tell it from the DMA target
    __shared__ int rdone[NCHAIN];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int ln = lane & 15;
    const int ntile = p.dv / DVT;
    long bh;
    int tile;
    int seg = 0;
    bool ident = false;  // identity-start columns (key channels j0 .. j0 + 31)
    if constexpr (!SEG) {
        // all column tiles of a head on one XCD (when the head count allows),
        // so that they share its L2 for the chunk records
        const long nbh = gridDim.x / ntile;
        if (nbh % kXcds == 0) {
            const long slot = blockIdx.x / kXcds;
            tile = static_cast<int>(slot % ntile);
            bh = (slot / ntile) * kXcds + blockIdx.x % kXcds;
        } else {
            bh = blockIdx.x / ntile;
            tile = static_cast<int>(blockIdx.x % ntile);
        }
    } else {
        // per head: segment 0's value tiles, then for each later segment its
        // value tiles and the DK / DVT identity tiles; all units of a head on
        // one XCD when the head count allows, as above
        const int per_seg = ntile + DK / DVT;
        const int units = ntile + (p.nseg - 1) * per_seg;
        const long nbh = gridDim.x / units;
        int u;
        if (nbh % kXcds == 0) {
            const long slot = blockIdx.x / kXcds;
            u = static_cast<int>(slot % units);
            bh = (slot / units) * kXcds + blockIdx.x % kXcds;
        } else {
            bh = blockIdx.x / units;
            u = static_cast<int>(blockIdx.x % units);
        }
        if (u < ntile) {
            tile = u;
        } else {
            seg = 1 + (u - ntile) / per_seg;
            const int r = (u - ntile) % per_seg;
            ident = r >= ntile;
            tile = ident ? r - ntile : r;
        }
    }
    const int j0 = tile * DVT;
    const long nc = p.nc;
    const long c0 = SEG ? seg * p.cps : 0;
    const long c1 = SEG ? min(c0 + p.cps, nc) : nc;
    const char* recs = p.rec + bh * nc * REC;
    const int slot0 = static_cast<int>(c0 % 3);  // part-A slot of chunk c0

    if (wave < NCHAIN) {
        f32x4 sacc[8];
        const int col = j0 + 16 * wave + ln;
        if (SEG && ident) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e) sacc[ib][e] = srow(ib, g, e) == col ? 1.0f : 0.0f;
        } else if (p.S0 && seg == 0) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e) sacc[ib][e] = p.S0[(bh * DK + srow(ib, g, e)) * p.dv + col];
        } else {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) sacc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        rdone[wave] = -1;
        __syncthreads();  // the first chunk is staged
        int sa = slot0;
        for (long c = c0; c < c1; ++c, sa = sa == 2 ? 0 : sa + 1) {
            const char* curA = smem + sa * PA;
            // part-B buffer; record offsets o >= PA are at curB + (o - PA)
            const char* curB = smem + L_B + (c & 1) * BUFB - PA;
            const uint16_t* kgh = reinterpret_cast<const uint16_t*>(curA + R_KGH);
            const uint16_t* kgl = reinterpret_cast<const uint16_t*>(curA + R_KGL);
            const uint16_t* qgh = reinterpret_cast<const uint16_t*>(curA + R_QGH);
            const uint16_t* qgl = reinterpret_cast<const uint16_t*>(curA + R_QGL);
            const uint16_t* kdh = reinterpret_cast<const uint16_t*>(curB + R_KDH);
            const uint16_t* kdl = reinterpret_cast<const uint16_t*>(curB + R_KDL);
            const float* sVt = reinterpret_cast<const float*>(curB + PA + B_VT) + (16 * wave + ln) * VTS;
            const float* gcs = reinterpret_cast<const float*>(curB + R_GC);

            // LDS reads are issued well ahead of their use: Kg first (it starts
            // the recurrence), then Qg, the transposed Kd and the fragments while
            // the Y products run
            auto rows = [&](const uint16_t* tile, int b, int t) {
                return *reinterpret_cast<const bf16x8*>(tile + kq_off(16 * b + ln, 32 * t + 8 * g));
            };
            bf16x8 ka[4][2][2];  // [k-step][row block][hi, lo]
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    ka[t][b][0] = rows(kgh, b, t);
                    ka[t][b][1] = rows(kgl, b, t);
                }
            bf16x8 bS[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) split_pair(sacc[2 * t], sacc[2 * t + 1], bS[t]);
            // Y = Kg S
            f32x4 y[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int b = 0; b < 2; ++b) y[b] = mfma32(ka[t][b][1], bS[t][0], y[b]);
#pragma unroll
                for (int b = 0; b < 2; ++b) y[b] = mfma32(ka[t][b][0], bS[t][1], y[b]);
#pragma unroll
                for (int b = 0; b < 2; ++b) y[b] = mfma32(ka[t][b][0], bS[t][0], y[b]);
            }
            bf16x8 qa[4][2][2];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    qa[t][b][0] = rows(qgh, b, t);
                    qa[t][b][1] = rows(qgl, b, t);
                }
            // Kd^T via transpose reads of the row-major tiles: lane ln of each 16
            // points at token 4g + ln / 4 and the 4 channels
            // 32 (ib / 2) + 4 (ib % 2) + 8 (ln % 4) .. + 3
            bf16x8 akh[8], akl[8];
            {
                const int tokA = 4 * g + (ln >> 2);
#pragma unroll
                for (int ib = 0; ib < 8; ++ib) {
                    const int pcol = 32 * (ib >> 1) + 4 * (ib & 1) + 8 * (ln & 3);
                    const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kdh + kq_off(tokA, pcol)));
                    const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kdh + kq_off(tokA + 16, pcol)));
                    const s16x4 l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kdl + kq_off(tokA, pcol)));
                    const s16x4 l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kdl + kq_off(tokA + 16, pcol)));
                    // whole-vector reinterpretation (an element-wise short -> bf16
                    // bit_cast loop is mis-lowered by this compiler)
                    akh[ib] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
                    akl[ib] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            }
            f32x4 gsc[8];
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) gsc[ib] = *reinterpret_cast<const f32x4*>(gcs + srow(ib, g, 0));
            auto a16 = [&](int sl, bf16x4 (&o)[2]) {
                o[0] = *reinterpret_cast<const bf16x4*>(curB + f16_off(sl, 0, lane));
                o[1] = *reinterpret_cast<const bf16x4*>(curB + f16_off(sl, 1, lane));
            };
            bf16x4 ad[2][2], an[2];
            a16(F16_D0, ad[0]);
            a16(F16_D1, ad[1]);
            a16(F16_N10, an);
            f32x4 vt[2];
#pragma unroll
            for (int R = 0; R < 2; ++R) vt[R] = *reinterpret_cast<const f32x4*>(sVt + 16 * R + 4 * g);
            bf16x8 ap[2][2];
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                ap[R][0] = *reinterpret_cast<const bf16x8*>(curB + pf_off(R, 0, lane));
                ap[R][1] = *reinterpret_cast<const bf16x8*>(curB + pf_off(R, 1, lane));
            }
            // keep the reads above the solve (the scheduler would otherwise sink
            // each one next to its first use and expose its latency)
            __builtin_amdgcn_sched_barrier(0);
            // this chunk's buffer is no longer read: the DMA wave may refill it
            // (the release store waits for the reads to return)
            __hip_atomic_store(&rdone[wave], static_cast<int>(c - c0), __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_WORKGROUP);

            // X = Vt - Y;  U_0 = D_0 X_0,  U_1 = D_1 X_1 - N U_0
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 W[2];
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                bf16x4 bx[2];
                split_d(vt[R] - y[R], bx);
                W[R] = mm22x16(ad[R], bx, zero);
            }
            bf16x4 bu0[2], bu1[2];
            split_d(W[0], bu0);
            const f32x4 u1 = mm22x16(an, bu0, W[1]);
            split_d(u1, bu1);
            bf16x8 bU[2];
            bU[0] = cat4(bu0[0], bu1[0]);
            bU[1] = cat4(bu0[1], bu1[1]);

            // S <- Diag(Gamma_31) S + Kd^T U
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) sacc[ib] *= gsc[ib];
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) sacc[ib] = mfma32(akl[ib], bU[0], sacc[ib]);
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) sacc[ib] = mfma32(akh[ib], bU[1], sacc[ib]);
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) sacc[ib] = mfma32(akh[ib], bU[0], sacc[ib]);

            // O = Qg S + P U, transposed (state / U as the A operand): lane (ln, g)
            // ends up with row 16R + ln, value columns 4g .. 4g + 3
            f32x4 oacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int b = 0; b < 2; ++b) oacc[b] = mfma32(bS[t][0], qa[t][b][1], oacc[b]);
#pragma unroll
                for (int b = 0; b < 2; ++b) oacc[b] = mfma32(bS[t][1], qa[t][b][0], oacc[b]);
#pragma unroll
                for (int b = 0; b < 2; ++b) oacc[b] = mfma32(bS[t][0], qa[t][b][0], oacc[b]);
            }
#pragma unroll
            for (int R = 0; R < 2; ++R) oacc[R] = mfma32(bU[0], ap[R][1], oacc[R]);
#pragma unroll
            for (int R = 0; R < 2; ++R) oacc[R] = mfma32(bU[1], ap[R][0], oacc[R]);
#pragma unroll
            for (int R = 0; R < 2; ++R) oacc[R] = mfma32(bU[0], ap[R][0], oacc[R]);
            if (SEG && ident) {
                const int c4 = j0 + 16 * wave + 4 * g;
#pragma unroll
                for (int R = 0; R < 2; ++R) {
                    const long tok = c * VC + 16 * R + ln;
                    if (tok < p.T) *reinterpret_cast<f32x4*>(p.qh + (bh * p.T + tok) * DK + c4) = oacc[R];
                }
            } else {
                const int c4 = j0 + 16 * wave + 4 * g;
#pragma unroll
                for (int R = 0; R < 2; ++R) {
                    const long tok = c * VC + 16 * R + ln;
                    if (tok >= p.T) continue;
                    const long oi = (bh * p.T + tok) * p.dv + c4;
                    if (p.o_bf16) {
                        uint2 pk;
                        pk.x = f32_to_bf16_bits(oacc[R][0]) | (static_cast<uint32_t>(f32_to_bf16_bits(oacc[R][1])) << 16);
                        pk.y = f32_to_bf16_bits(oacc[R][2]) | (static_cast<uint32_t>(f32_to_bf16_bits(oacc[R][3])) << 16);
                        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + oi) = pk;
                    } else {
                        *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + oi) = oacc[R];
                    }
                }
            }
            __syncthreads();
        }
        if constexpr (SEG) {
            // the segment's end state: value columns, or the transition
            const long sb = (bh * p.nseg + seg) * DK;
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (ident) p.phi[(sb + srow(ib, g, e)) * DK + col] = sacc[ib][e];
                    else p.nst[(sb + srow(ib, g, e)) * p.dv + col] = sacc[ib][e];
                }
        } else if (p.ST) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e) p.ST[(bh * DK + srow(ib, g, e)) * p.dv + col] = sacc[ib][e];
        }
        return;
    }

    if (wave == NCHAIN) {
        // wave 2: the records, HBM -> LDS by DMA (16 bytes per lane, 1 KiB per
        // instruction, a straight copy), two chunks ahead.  In chunk c it
        // fetches chunk c + 2: part A at once (into chunk c - 1's slot), part B
        // as soon as both chain waves have read chunk c's buffer.  At the
        // barrier that ends chunk c only chunk c + 1 must have landed: the wait
        // leaves chunk c + 2's REC / 1024 loads in flight (the barrier is
        // issued without the workgroup fence, which would wait for all of them).
        constexpr int NL = REC / 1024;
        static_assert(NL <= 63, "one record's loads fit the load counter");
        static_assert(NCHAIN == 2, "the flag test below reads two chain waves");
        auto dma = [&](long c, int off, int bytes, char* dst) {
            const char* src = recs + c * REC + off + 16 * lane;
#pragma unroll 8
            for (int m = 0; m < bytes / 1024; ++m)
                __builtin_amdgcn_global_load_lds((const void*)(src + m * 1024),
                                                 (__attribute__((address_space(3))) void*)(dst + m * 1024), 16, 0, 0);
        };
        auto dma_a = [&](long c, int slot) { dma(c, 0, PA, smem + slot * PA); };
        auto dma_b = [&](long c) { dma(c, PA, PB, smem + L_B + (c & 1) * BUFB); };
        // s_waitcnt immediates (gfx9 layout: vmcnt bits 3:0 and 15:14,
        // expcnt 6:4, lgkmcnt 11:8): vmcnt(NL) and vmcnt(0), the others free
        constexpr int WAIT_NL = ((NL >> 4) << 14) | (NL & 15) | (7 << 4) | (15 << 8);
        constexpr int WAIT_0 = (7 << 4) | (15 << 8);
        auto barrier_after = [&](bool more) {
            if (more) __builtin_amdgcn_s_waitcnt(WAIT_NL);
            else __builtin_amdgcn_s_waitcnt(WAIT_0);
            __builtin_amdgcn_s_barrier();
        };
        // A chain wave's flag, read with its own wait: a compiler-generated LDS
        // read here would first wait for every DMA in flight (it cannot tell
        // the flag from the DMA targets).
        auto flag = [&](int w) {
            int v;
            const unsigned a = static_cast<unsigned>(
                reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const int*)(&rdone[w])));
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
            return v;
        };
        const int s1 = slot0 == 2 ? 0 : slot0 + 1;
        if (c0 < c1) {
            dma_a(c0, slot0);
            dma_b(c0);
        }
        if (c0 + 1 < c1) {
            dma_a(c0 + 1, s1);
            dma_b(c0 + 1);
        }
        barrier_after(c0 + 1 < c1);
        int s2 = s1 == 2 ? 0 : s1 + 1;  // slot of chunk c + 2
        for (long c = c0; c < c1; ++c, s2 = s2 == 2 ? 0 : s2 + 1) {
            const bool more = c + 2 < c1;
            if (more) {
                dma_a(c + 2, s2);
                // both chain waves are past their reads of chunk c (they set the
                // flag before the barrier that ends chunk c, so this ends)
                const int want = static_cast<int>(c - c0);
                while (min(flag(0), flag(1)) < want) __builtin_amdgcn_s_sleep(1);
                dma_b(c + 2);
            }
            barrier_after(more);
        }
    } else {
        // wave 3: value tile of a chunk, scaled by sqrt(gamma), gamma or 1, transposed:
        // lane (ln, g) holds tokens 2 ln, 2 ln + 1 of columns j0 + 8g .. + 7.
        // Registers are refilled one chunk ahead; rows past T get 0.
        uint4 vr[2] = {};
        f32x4 gv[2][2] = {};
        float gs[2] = {0.0f, 0.0f};
        auto load = [&](long c) {
            if (SEG && ident) return;  // no values (and j0 indexes key channels, not value columns)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const long r = bh * p.T + min(c * VC + 2 * ln + i, p.T - 1);
                vr[i] = *reinterpret_cast<const uint4*>(p.v + r * p.dv + j0 + 8 * g);
                if (p.gvec) {
                    gv[i][0] = *reinterpret_cast<const f32x4*>(p.gsrc + r * p.gts + j0 + 8 * g);
                    gv[i][1] = *reinterpret_cast<const f32x4*>(p.gsrc + r * p.gts + j0 + 8 * g + 4);
                } else {
                    gs[i] = p.gsrc[r * p.gts];
                }
            }
        };
        auto stage = [&](long c, char* buf) {
            float* sVt = reinterpret_cast<float*>(buf + B_VT);  // a part-B buffer
            bool okt[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) okt[i] = c * VC + 2 * ln + i < p.T;
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                f32x2 v2;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const float gam = p.gvec ? gv[i][cc >> 2][cc & 3] : gs[i];
                    const float sc = p.vmode == VAL_SQRT_GAIN ? sqrt_hw(gam) : (p.vmode == VAL_GAIN ? gam : 1.0f);
                    v2[i] = (okt[i] && !(SEG && ident)) ? bf16_at(vr[i], cc) * sc : 0.0f;
                }
                *reinterpret_cast<f32x2*>(sVt + (8 * g + cc) * VTS + 2 * ln) = v2;
            }
        };
        if (c0 < c1) {
            load(c0);
            stage(c0, smem + L_B + (c0 & 1) * BUFB);
            if (c0 + 1 < c1) load(c0 + 1);
        }
        __syncthreads();
        for (long c = c0; c < c1; ++c) {
            if (c + 1 < c1) {
                stage(c + 1, smem + L_B + ((c + 1) & 1) * BUFB);
                if (c + 2 < c1) load(c + 2);
            }
            __syncthreads();
        }
    }
}

}  // namespace
}  // namespace pdn
