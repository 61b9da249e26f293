// Prefill for per-channel decay and gains and the diagonal preconditioner
// (KDA / FG^2-GDN / Gated DeltaNet-2 gating), bf16 q/k/v, dk = 128.
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
#include "chunk_tile.h"
#include "kernels.h"

namespace pdn {
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
// preconditioner pre-pass
// ---------------------------------------------------------------------------

// Sum of k (.) k over each chunk: one wave per (b, h, chunk), four chunks per
// workgroup.  Lane (ln, g) reads channels 8 ln .. 8 ln + 7 (16 bytes) of the
// tokens 4s + g, s = 0..7; the four token groups are then added across lanes.
constexpr int KSQ_NTHR = 256;
__global__ void __launch_bounds__(KSQ_NTHR) vec_ksq_kernel(const uint16_t* k, float* ks, long T, long nc, long nid) {
    const int lane = threadIdx.x & 63;
    const long id = blockIdx.x * (KSQ_NTHR / 64L) + (threadIdx.x >> 6);
    if (id >= nid) return;
    const long bh = id / nc;
    const long t0 = (id % nc) * VC;
    const int ln = lane & 15, g = lane >> 4;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // every row is loaded (rows past T reread the last one) before any is
    // used, and rows past T are masked afterwards: a load behind the test
    // would make the compiler wait for each row in turn
    uint4 u[VC / 4];
#pragma unroll
    for (int s4 = 0; s4 < VC / 4; ++s4)
        u[s4] = *reinterpret_cast<const uint4*>(k + (bh * T + min(t0 + 4 * s4 + g, T - 1)) * DK + 8 * ln);
#pragma unroll
    for (int s4 = 0; s4 < VC / 4; ++s4) {
        const float m = t0 + 4 * s4 + g < T ? 1.0f : 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = bf16_at(u[s4], j) * m;
            acc[j] = fmaf(x, x, acc[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        acc[j] += __shfl_xor(acc[j], 16, 64);
        acc[j] += __shfl_xor(acc[j], 32, 64);
    }
    if (g == 0) {
        float* dst = ks + id * DK + 8 * ln;
        *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
}

// Exclusive running sum over the chunks of each (b, h), in place, starting
// from A0; the total goes to AT.  One workgroup per (b, h, 32 channels):
// thread (segment, channel) sums its run of chunks, the segment totals are
// prefixed through LDS, and a second pass writes the running values.  Each
// thread's run is a chain of dependent loads, so the runs are kept short
// (32 segments per head).
constexpr int KSCAN_SEG = 32;
constexpr int KSCAN_CH = 32;
__global__ void __launch_bounds__(KSCAN_SEG * KSCAN_CH) vec_kscan_kernel(float* ks, const float* A0, float* AT, long nc) {
    __shared__ float tot[KSCAN_SEG][KSCAN_CH];
    const long bh = blockIdx.x / (DK / KSCAN_CH);
    const int ci = threadIdx.x % KSCAN_CH;
    const int i = static_cast<int>(blockIdx.x % (DK / KSCAN_CH)) * KSCAN_CH + ci;
    const int sg = threadIdx.x / KSCAN_CH;
    const long len = (nc + KSCAN_SEG - 1) / KSCAN_SEG;
    const long c0 = min(sg * len, nc), c1 = min(c0 + len, nc);
    float* col = ks + bh * nc * DK + i;
    float sum = 0.0f;
    long c = c0;
    for (; c + 8 <= c1; c += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = col[(c + u) * DK];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; c < c1; ++c) sum += col[c * DK];
    tot[sg][ci] = sum;
    __syncthreads();
    float run = A0 ? A0[bh * DK + i] : 0.0f;
    for (int q = 0; q < sg; ++q) run += tot[q][ci];
    c = c0;
    for (; c + 8 <= c1; c += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = col[(c + u) * DK];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            col[(c + u) * DK] = run;
            run += v[u];
        }
    }
    for (; c < c1; ++c) {
        const float v = col[c * DK];
        col[c * DK] = run;
        run += v;
    }
    if (AT && sg == KSCAN_SEG - 1) AT[bh * DK + i] = run;
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

// ---------------------------------------------------------------------------
// sequence segments: combining the segments' end states, correcting outputs
// ---------------------------------------------------------------------------

// The recurrence is linear in (state, values): a segment run from start
// state S has end state Phi S + N and outputs o_t + (Phi_t^T q_t)^T S, with
// N, o_t from the run with S = 0 and Phi, Phi_t^T q_t from the identity-start
// columns.  The segments' start states follow S_1 = N_0 (segment 0 ran from
// the real start state), S_{g+1} = Phi_g S_g + N_g; every column of the state
// follows its own recurrence, so one workgroup takes one (head, 32-column
// tile) through all segments.  It stores each S_g (g >= 1) for the output
// correction and writes the final state.  Products are fp32 16x16x4 MFMAs
// (exact fp32 products, fp32 accumulation).
constexpr int SEG_NTHR = 256;
constexpr int CT = 32;  // state columns per combine workgroup
__global__ void __launch_bounds__(SEG_NTHR) vec_seg_combine_kernel(const float* nst, const float* phi,
                                                                   float* sst, float* ST, int nseg, int dv) {
    __shared__ float sPhi[DK][DK + 4];
    __shared__ float sS[DK][CT + 16];  // row stride 48: the four k rows a read touches fall in distinct banks
    const int ntile = dv / CT;
    const long bh = blockIdx.x / ntile;
    const int j0 = (blockIdx.x % ntile) * CT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    const float* nb = nst + bh * nseg * DK * dv;
    float* sb = sst + bh * nseg * DK * dv;
    // S_1 = N_0 (columns j0 .. j0 + CT - 1)
    for (int i = tid; i < DK * CT; i += SEG_NTHR) sS[i / CT][i % CT] = nb[(i / CT) * dv + j0 + i % CT];
    for (int g = 1;; ++g) {
        __syncthreads();
        // S_g is in sS: keep it for the correction (g < nseg) or it is the
        // final state (g == nseg)
        float* dst = g < nseg ? sb + g * DK * dv : (ST ? ST + bh * DK * dv : nullptr);
        if (dst)
            for (int i = tid; i < DK * CT; i += SEG_NTHR) dst[(i / CT) * dv + j0 + i % CT] = sS[i / CT][i % CT];
        if (g == nseg) break;
        // S_{g+1} = Phi_g S_g + N_g
        const float* P = phi + (bh * nseg + g) * DK * DK;
        for (int i = tid; i < DK * DK; i += SEG_NTHR) sPhi[i / DK][i % DK] = P[i];
        __syncthreads();
        // wave w: rows 32w .. 32w + 31 (two 16-row blocks) x 32 columns (two blocks)
        f32x4 acc[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[rb][cb][e] = nb[(g * DK + 32 * wave + 16 * rb + 4 * g4 + e) * dv + j0 + 16 * cb + ln];
        for (int k = 0; k < DK; k += 4) {
            float a[2], b[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) a[rb] = sPhi[32 * wave + 16 * rb + ln][k + g4];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) b[cb] = sS[k + g4][16 * cb + ln];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma4(a[rb], b[cb], acc[rb][cb]);
        }
        __syncthreads();  // every wave has read S_g
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) sS[32 * wave + 16 * rb + 4 * g4 + e][16 * cb + ln] = acc[rb][cb][e];
    }
}

// o_t += (Phi_t^T q_t)^T S_g for the tokens of segments g >= 1: one workgroup
// per (head, segment, 256-token tile).  For each pass of 128 state columns,
// S_g^T is staged in LDS as bf16 hi/lo terms (row = state column, its 128
// channels; 16-byte chunks XOR-swizzled by the row so that the 16 rows an
// operand read touches fall in distinct banks).  Each wave takes 16-token
// blocks; per block the transposed product out^T = S_g^T qh^T runs as
// 16x16x32 bf16 MFMAs on hi/lo terms (hi.hi + hi.lo + lo.hi, fp32
// accumulation), so that lane (ln, g) ends with token ln, columns 4g .. 4g + 3
// of each 16-column block and updates o in 16-byte pieces.
//
// With two segments (the usual split) S_1 is segment 0's end state N_0 itself,
// so the correction reads it from there (`direct`) and needs no combine pass;
// the launch then also holds one workgroup per (head, CT state columns) that
// forms the final state S_T = Phi_1 N_0 + N_1 (two_seg_final_state), beside
// the correction workgroups.
constexpr int COR_TOK = 256;
constexpr int COR_CB = 128;
__device__ __forceinline__ int cor_off(int row, int ch) {  // bf16 element offset in a staged tile
    return row * DK + ((((ch >> 3) ^ (row & 15)) << 3) | (ch & 7));
}

// S_T = Phi_1 N_0 + N_1 for columns j0 .. j0 + CT - 1 of head bh (two
// segments), fp32 16x16x4 MFMAs as in the combine pass; the key dimension in
// two halves of 64 so that Phi's half (row stride 68) and N_0's rows (stride
// 48) fit in the correction's LDS.
__device__ __forceinline__ void two_seg_final_state(const float* nst, const float* phi, float* ST, long bh,
                                                    int j0, int dv, float* fbuf) {
    constexpr int KH = DK / 2;
    float(*sPhi)[KH + 4] = reinterpret_cast<float(*)[KH + 4]>(fbuf);
    float(*sS)[CT + 16] = reinterpret_cast<float(*)[CT + 16]>(fbuf + DK * (KH + 4));
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    const float* N0 = nst + (bh * 2) * DK * dv;
    const float* N1 = N0 + DK * dv;
    const float* P = phi + (bh * 2 + 1) * DK * DK;
    // wave w: rows 32w .. 32w + 31 (two 16-row blocks) x CT = 32 columns (two blocks)
    f32x4 acc[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[rb][cb][e] = N1[(32 * wave + 16 * rb + 4 * g4 + e) * dv + j0 + 16 * cb + ln];
    for (int kh = 0; kh < DK; kh += KH) {
        // every load of the half before its LDS stores (a store after each
        // load would wait for it)
        constexpr int NP = DK * KH / 4 / SEG_NTHR, NS = KH * CT / 4 / SEG_NTHR;
        static_assert(NP * SEG_NTHR == DK * KH / 4 && NS * SEG_NTHR == KH * CT / 4, "whole passes");
        f32x4 pv[NP], sv[NS];
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int i = tid + u * SEG_NTHR, r = i / (KH / 4), c4 = i % (KH / 4);
            pv[u] = *reinterpret_cast<const f32x4*>(P + r * DK + kh + 4 * c4);
        }
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int i = tid + u * SEG_NTHR, r = i / (CT / 4), c4 = i % (CT / 4);
            sv[u] = *reinterpret_cast<const f32x4*>(N0 + (kh + r) * dv + j0 + 4 * c4);
        }
        __syncthreads();  // the previous half has been read
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int i = tid + u * SEG_NTHR, r = i / (KH / 4), c4 = i % (KH / 4);
            *reinterpret_cast<f32x4*>(&sPhi[r][4 * c4]) = pv[u];
        }
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int i = tid + u * SEG_NTHR, r = i / (CT / 4), c4 = i % (CT / 4);
            *reinterpret_cast<f32x4*>(&sS[r][4 * c4]) = sv[u];
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < KH; k += 4) {
            float a[2], b[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) a[rb] = sPhi[32 * wave + 16 * rb + ln][k + g4];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) b[cb] = sS[k + g4][16 * cb + ln];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma4(a[rb], b[cb], acc[rb][cb]);
        }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ST[(bh * DK + 32 * wave + 16 * rb + 4 * g4 + e) * dv + j0 + 16 * cb + ln] = acc[rb][cb][e];
}

__global__ void __launch_bounds__(SEG_NTHR, 2) vec_seg_correct_kernel(const float* qh, const float* sst, const float* nst,
                                                                   const float* phi, float* ST, float* o, long T,
                                                                   int nseg, long seg_tokens, int dv,
                                                                   long tiles_per_seg, long ncorr) {
    __shared__ __attribute__((aligned(16))) uint16_t sbuf[2 * COR_CB * DK];
    uint16_t* sH = sbuf;
    uint16_t* sL = sbuf + COR_CB * DK;
    const bool direct = nseg == 2;  // S_1 = N_0: read segment 0's end state
    if (blockIdx.x >= ncorr) {      // two segments: a final-state workgroup
        const long u = blockIdx.x - ncorr;
        two_seg_final_state(nst, phi, ST, u / (dv / CT), static_cast<int>(u % (dv / CT)) * CT, dv,
                            reinterpret_cast<float*>(sbuf));
        return;
    }
    const long unit = blockIdx.x;
    const long per_bh = (nseg - 1) * tiles_per_seg;
    const long bh = unit / per_bh;
    const int gs = 1 + static_cast<int>((unit % per_bh) / tiles_per_seg);
    const long tile = (unit % per_bh) % tiles_per_seg;
    const long t0 = gs * seg_tokens + tile * COR_TOK;
    const long t1 = min(min(t0 + COR_TOK, (gs + 1) * seg_tokens), T);
    if (t0 >= t1) return;  // whole workgroup
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, g = lane >> 4;
    const float* S = direct ? nst + (bh * nseg) * DK * dv : sst + (bh * nseg + gs) * DK * dv;
    for (int jb = 0; jb < dv; jb += COR_CB) {
        const int nj = min(COR_CB, dv - jb);  // a multiple of 32
        // stage S_g^T (columns jb .. jb + nj) as hi/lo bf16: item (column c,
        // channels 8m .. 8m + 7), consecutive threads on consecutive columns;
        // every load first (columns past nj reread column jb and are zeroed)
        constexpr int NIT = COR_CB * (DK / 8) / SEG_NTHR;
        static_assert(NIT * SEG_NTHR == COR_CB * (DK / 8), "whole passes");
        float x[NIT][8];
#pragma unroll
        for (int u = 0; u < NIT; ++u) {
            const int it = tid + u * SEG_NTHR, c = it % COR_CB, m = it / COR_CB;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[u][e] = S[(8 * m + e) * dv + jb + (c < nj ? c : 0)];
        }
        __syncthreads();  // the previous pass is done with the staged tile
#pragma unroll
        for (int u = 0; u < NIT; ++u) {
            const int it = tid + u * SEG_NTHR, c = it % COR_CB, m = it / COR_CB;
            const float keep = c < nj ? 1.0f : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[u][e] *= keep;
            uint4 h, l;
            split8(x[u], h, l);
            *reinterpret_cast<uint4*>(sH + cor_off(c, 8 * m)) = h;
            *reinterpret_cast<uint4*>(sL + cor_off(c, 8 * m)) = l;
        }
        __syncthreads();
        for (long tb = t0 + 16 * wave; tb < t1; tb += 64) {
            const long tok = tb + ln;  // this lane's token (B operand column)
            const bool tv = tok < t1;
            const float* qrow = qh + (bh * T + (tv ? tok : t1 - 1)) * DK;
            // B operands: qh row `tok`, channels 32 t + 8 g .. + 7, hi/lo
            bf16x8 bh_[4], bl_[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 a0 = *reinterpret_cast<const f32x4*>(qrow + 32 * t + 8 * g);
                const f32x4 a1 = *reinterpret_cast<const f32x4*>(qrow + 32 * t + 8 * g + 4);
                bf16x8 hl[2];
                split_pair(a0, a1, hl);
                bh_[t] = hl[0];
                bl_[t] = hl[1];
            }
            // this lane's outputs, all read before the products (a read behind
            // the token test would be waited for one at a time); past t1 the
            // last token is read again and not written
            float* orow = o + (bh * T + (tv ? tok : t1 - 1)) * dv + jb + 4 * g;
            const int ncb = nj / 16;
            f32x4 ov[COR_CB / 16];
#pragma unroll
            for (int cb = 0; cb < COR_CB / 16; ++cb)
                ov[cb] = *reinterpret_cast<const f32x4*>(orow + 16 * min(cb, ncb - 1));
#pragma unroll
            for (int cb = 0; cb < COR_CB / 16; ++cb) {
                if (cb >= ncb) break;
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(sH + cor_off(16 * cb + ln, 32 * t + 8 * g));
                    const bf16x8 al = *reinterpret_cast<const bf16x8*>(sL + cor_off(16 * cb + ln, 32 * t + 8 * g));
                    acc = mfma32(al, bh_[t], acc);
                    acc = mfma32(ah, bl_[t], acc);
                    acc = mfma32(ah, bh_[t], acc);
                }
                // acc: token ln, state columns 16 cb + 4 g .. + 3
                if (tv) *reinterpret_cast<f32x4*>(orow + 16 * cb) = ov[cb] + acc;
            }
        }
    }
}

bool vec_gates(const pdn_chunk_fwd_args& a) {
    return a.alpha_mode == PDN_ALPHA_VEC || a.beta_mode == PDN_GATE_VEC || a.precond_eps >= 0.0f;
}

long num_chunks(const pdn_chunk_fwd_args& a) { return (static_cast<long>(a.T) + VC - 1) / VC; }

template <bool AVEC, bool BVEC, bool PRE, bool STAB>
void launch_prep_km(const PrepParams& pp, int km, long nblk, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(nblk)), block(256);
    if (km == PDN_KEY_ERASE_GATE) vec_prep_kernel<AVEC, BVEC, PRE, PDN_KEY_ERASE_GATE, STAB><<<grid, block, 0, stream>>>(pp);
    else if (km == PDN_KEY_WRITE_GATE) vec_prep_kernel<AVEC, BVEC, PRE, PDN_KEY_WRITE_GATE, STAB><<<grid, block, 0, stream>>>(pp);
    else vec_prep_kernel<AVEC, BVEC, PRE, PDN_KEY_SYMMETRIC, STAB><<<grid, block, 0, stream>>>(pp);
}
// the stabilised coefficient is a separate instantiation so that it costs the
// other modes no registers
template <bool AVEC, bool BVEC, bool PRE>
void launch_prep(const PrepParams& pp, int km, bool stab, long nblk, hipStream_t stream) {
    if constexpr (PRE) {
        if (stab) {
            launch_prep_km<AVEC, BVEC, PRE, true>(pp, km, nblk, stream);
            return;
        }
    }
    launch_prep_km<AVEC, BVEC, PRE, false>(pp, km, nblk, stream);
}

}  // namespace

// Sequence segments for few-head prefills: as many as fit one wave of chain
// workgroups (one per CU), at least 8 chunks each, at most 8; fp32 output only
// (the correction adds to the stored outputs).  The slot count is the MI355X
// CU count as a constant, not a device query: the segment count sets the
// workspace size, which a caller may ask for before any device is current.
constexpr long kChainSlots = 256;
int vec_segments(const pdn_chunk_fwd_args& a) {
    if (a.o_dtype != PDN_F32) return 1;
    const long nbh = static_cast<long>(a.B) * a.H, nc = num_chunks(a);
    const long vt = a.dv / DVT, it = DK / DVT;
    int G = 1;
    for (int g = 2; g <= 8; ++g) {
        if (nc < 8L * g || nbh * (vt * g + it * (g - 1)) > kChainSlots) break;
        G = g;
    }
    return G;
}

// workspace pieces after the chunk records (and the k.k sums)
struct SegBufs {
    size_t qh, nst, phi, sst, end;
};
SegBufs seg_layout(const pdn_chunk_fwd_args& a, size_t start, int G) {
    const size_t nbh = static_cast<size_t>(a.B) * a.H;
    SegBufs b;
    b.qh = start;
    b.nst = b.qh + (G > 1 ? nbh * a.T * DK * sizeof(float) : 0);
    b.phi = b.nst + (G > 1 ? nbh * G * DK * a.dv * sizeof(float) : 0);
    b.sst = b.phi + (G > 1 ? nbh * G * DK * DK * sizeof(float) : 0);
    b.end = b.sst + (G > 1 ? nbh * G * DK * a.dv * sizeof(float) : 0);
    return b;
}

bool chunk_vec_supported(const pdn_chunk_fwd_args& a) {
    return a.qkv_dtype == PDN_BF16 && a.dk == DK && a.dv % DVT == 0 &&
           (vec_gates(a) || a.key_mode != PDN_KEY_SYMMETRIC);
}

size_t chunk_vec_workspace_bytes(const pdn_chunk_fwd_args& a) {
    const long nrec = static_cast<long>(a.B) * a.H * num_chunks(a);
    size_t n = static_cast<size_t>(nrec) * REC;
    if (a.precond_eps >= 0.0f) n += static_cast<size_t>(nrec) * DK * sizeof(float);
    return seg_layout(a, n, vec_segments(a)).end;
}

hipError_t launch_chunk_vec(const pdn_chunk_fwd_args& a, hipStream_t stream) {
    const long nbh = static_cast<long>(a.B) * a.H;
    const long nc = num_chunks(a);
    char* ws = static_cast<char*>(a.workspace);
    const bool pre = a.precond_eps >= 0.0f;
    float* ksum = pre ? reinterpret_cast<float*>(ws + static_cast<size_t>(nbh * nc) * REC) : nullptr;
    if (pre) {
        const long nid = nbh * nc;
        vec_ksq_kernel<<<dim3(static_cast<unsigned>((nid + 3) / 4)), dim3(KSQ_NTHR), 0, stream>>>(
            static_cast<const uint16_t*>(a.k), ksum, a.T, nc, nid);
        vec_kscan_kernel<<<dim3(static_cast<unsigned>(nbh * (DK / KSCAN_CH))), dim3(KSCAN_SEG * KSCAN_CH), 0, stream>>>(
            ksum, a.precond_A0, a.precond_AT, nc);
    }
    PrepParams pp;
    pp.q = static_cast<const uint16_t*>(a.q);
    pp.k = static_cast<const uint16_t*>(a.k);
    pp.has_alpha = a.alpha_mode != PDN_ALPHA_NONE;
    pp.log_alpha = a.log_alpha;
    pp.beta = a.beta;
    pp.astart = ksum;
    pp.rec = ws;
    pp.T = a.T;
    pp.nc = nc;
    pp.nbh = nbh;
    pp.eps = pre ? a.precond_eps : 0.0f;
    const bool stab = pre && a.precond_mode == PDN_PRECOND_STABILISED;
    pp.l2x = stab ? std::log2(a.precond_x) : 0.0f;
    const long nblk = (nbh * nc + 3) / 4;
    const bool avec = a.alpha_mode == PDN_ALPHA_VEC, bvec = a.beta_mode == PDN_GATE_VEC;
    const int km = a.key_mode;
    if (avec) {
        if (bvec) pre ? launch_prep<true, true, true>(pp, km, stab, nblk, stream) : launch_prep<true, true, false>(pp, km, stab, nblk, stream);
        else pre ? launch_prep<true, false, true>(pp, km, stab, nblk, stream) : launch_prep<true, false, false>(pp, km, stab, nblk, stream);
    } else {
        if (bvec) pre ? launch_prep<false, true, true>(pp, km, stab, nblk, stream) : launch_prep<false, true, false>(pp, km, stab, nblk, stream);
        else pre ? launch_prep<false, false, true>(pp, km, stab, nblk, stream) : launch_prep<false, false, false>(pp, km, stab, nblk, stream);
    }

    ChainParams cp;
    cp.v = static_cast<const uint16_t*>(a.v);
    cp.rec = ws;
    if (a.gamma_mode == PDN_GATE_VEC) {
        cp.gsrc = a.gamma; cp.gts = a.dv; cp.gvec = 1;
    } else if (a.gamma_mode == PDN_GATE_SCALAR) {
        cp.gsrc = a.gamma; cp.gts = 1; cp.gvec = 0;
    } else if (a.beta_mode == PDN_GATE_VEC) {  // raw beta, dk == dv
        cp.gsrc = a.beta; cp.gts = a.dk; cp.gvec = 1;
    } else {
        cp.gsrc = a.beta; cp.gts = 1; cp.gvec = 0;
    }
    if (a.key_mode == PDN_KEY_SYMMETRIC) cp.vmode = VAL_SQRT_GAIN;
    else if (a.key_mode == PDN_KEY_WRITE_GATE && a.gamma_mode == PDN_GAMMA_SAME_AS_BETA) cp.vmode = VAL_UNIT;
    else cp.vmode = VAL_GAIN;
    cp.S0 = a.S0;
    cp.ST = a.ST;
    cp.o = a.o;
    cp.T = a.T;
    cp.nc = nc;
    cp.dv = a.dv;
    cp.o_bf16 = a.o_dtype == PDN_BF16;
    const int G = vec_segments(a);
    const long vt = a.dv / DVT, it = DK / DVT;
    size_t recs_end = static_cast<size_t>(nbh * nc) * REC;
    if (pre) recs_end += static_cast<size_t>(nbh * nc) * DK * sizeof(float);
    const SegBufs sb = seg_layout(a, recs_end, G);
    cp.nseg = G;
    cp.cps = G > 1 ? (nc + G - 1) / G : nc;
    cp.qh = reinterpret_cast<float*>(ws + sb.qh);
    cp.nst = reinterpret_cast<float*>(ws + sb.nst);
    cp.phi = reinterpret_cast<float*>(ws + sb.phi);
    const long nwg = nbh * (vt + (G - 1) * (vt + it));
    if (G > 1) vec_chain_kernel<true><<<dim3(static_cast<unsigned>(nwg)), dim3(NTHR), 0, stream>>>(cp);
    else vec_chain_kernel<false><<<dim3(static_cast<unsigned>(nwg)), dim3(NTHR), 0, stream>>>(cp);
    if (G > 1)
        return launch_seg_finish(cp.nst, cp.phi, reinterpret_cast<float*>(ws + sb.sst), a.ST, cp.qh,
                                 static_cast<float*>(a.o), nbh, a.T, G, cp.cps * VC, a.dv, stream);
    return hipGetLastError();
}

hipError_t launch_seg_finish(const float* nst, const float* phi, float* sst, float* ST, const float* qh,
                             float* o, long nbh, long T, int nseg, long seg_tokens, int dv,
                             hipStream_t stream) {
    const long tiles = (seg_tokens + COR_TOK - 1) / COR_TOK;
    const long ncorr = nbh * (nseg - 1) * tiles;
    long nfinal = 0;
    if (nseg == 2) {
        // no combine pass: the final state comes from extra workgroups of the
        // correction launch (none without ST)
        nfinal = ST ? nbh * (dv / CT) : 0;
    } else {
        vec_seg_combine_kernel<<<dim3(static_cast<unsigned>(nbh * (dv / CT))), dim3(SEG_NTHR), 0, stream>>>(
            nst, phi, sst, ST, nseg, dv);
    }
    vec_seg_correct_kernel<<<dim3(static_cast<unsigned>(ncorr + nfinal)), dim3(SEG_NTHR), 0, stream>>>(
        qh, sst, nst, phi, ST, o, T, nseg, seg_tokens, dv, tiles, ncorr);
    return hipGetLastError();
}

}  // namespace pdn
