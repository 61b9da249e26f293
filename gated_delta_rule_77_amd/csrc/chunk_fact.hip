// Prefill for per-token scalar decay and gain (Gated DeltaNet / DeltaNet
// gating), bf16 q/k/v, dk = 128: the throughput path.
//
// Same chunk algebra as chunk_fwd.hip, over whole 64-token chunks ("Gated
// DeltaNet-2" method section 3: decay absorbed into the erase/write matrices,
// one unit-lower-triangular solve per chunk).  With G_r the cumulative log
// decay from the chunk start, Gamma_r = exp(G_r), sb_r = sqrt(beta_r):
//
//   T_rs = sb_r sb_s exp(G_r - G_s) (k_r . k_s)      s < r
//   P_rs = sb_s exp(G_r - G_s) (q_r . k_s)           s <= r
//   X    = Vt - diag(sb Gamma) K S
//   U    = (I + T)^-1 X
//   O    = diag(Gamma) Q S + P U
//   S   <- Gamma_63 S + K^T diag(sb exp(G_63 - G)) U
//
// U is found by block forward substitution over the four 16-token blocks of
// the chunk: U_R = D_R X_R - sum_{J<R} N_RJ U_J with D_R = (I + T_RR)^-1 and
// N_RJ = D_R T_RJ, so the only dependent steps are the three N products.
//
// Work split.  A workgroup owns (b, h, 32 value columns) for the whole
// sequence and has four waves:
//   waves 0-1 ("chain"): 16 state columns each, held in MFMA accumulator
//     registers; all products on hi/lo bf16 operands with fp32 accumulation.
//   waves 2-3 ("helpers"): while the chain waves work on chunk c, they build
//     everything chunk c+1 needs from registers loaded one chunk ahead:
//     wave 2 stages the key tile, forms T with MFMAs and inverts its 16x16
//     diagonal blocks by forward substitution; wave 3 stages the query tile,
//     the gain-scaled value tile and the per-row scales, and forms P.  The
//     blocks of D, N and P are written already split into bf16 hi/lo
//     fragments in the per-lane order of the chain's MFMA operands, so the
//     chain reads them with one LDS load per term and no conversion.
// LDS holds two chunk buffers; one workgroup barrier per chunk hands a
// buffer from the helpers to the chain waves.  The state-update operand K^T
// is read from the row-major key tile with the gfx950 LDS transpose read
// (ds_read_b64_tr_b16), so no transposed copy of K is stored.
#include <type_traits>

#include "chunk_tile.h"
#include "kernels.h"

namespace pdn {
namespace {

using namespace tile;

constexpr int CH = 64;
constexpr int NCHAIN = 2;
constexpr int NTHR = 64 * (NCHAIN + 2);
constexpr int DVT = 16 * NCHAIN;
constexpr int VTS = CH + 4;  // row stride of the transposed value tile (floats)
constexpr int NFRAG = 6;     // lower-triangular (block row, k-step) fragments of P

// Solve fragments (hi and lo terms, per lane): two 16x32 operands [-N_R0 | -N_R1]
// for R = 2, 3 (16 bytes per lane and term), then six 16x16 operands D_0..D_3,
// -N_10, -N_32 (8 bytes per lane and term).
constexpr int TF16 = 2 * 2 * 64 * 16;
constexpr int TF_BYTES = TF16 + 6 * 2 * 64 * 8;
enum { F32_N2 = 0, F32_N3 = 1 };
enum { F16_D0 = 0, F16_N10 = 4, F16_N32 = 5 };

// LDS layout (bytes).  Three key tiles (bf16 [64][128], swizzled; chunk c in
// slot c % 3: the chain reads chunk c while the helpers read chunk c + 1 and
// wave 2 stages chunk c + 2), then two per-parity buffers holding the query
// tile, solve and P fragments, the value tile transposed (fp32 [32][VTS]) and
// the per-row scales.
constexpr int KTILE = CH * DK * 2;
constexpr int B_Q = 0;
constexpr int B_TF = B_Q + CH * DK * 2;
constexpr int B_PF = B_TF + TF_BYTES;
constexpr int B_VT = B_PF + NFRAG * 2 * 64 * 16;
constexpr int B_SC = B_VT + DVT * VTS * 4;
constexpr int BUF = B_SC + 4 * CH * 4;  // rsKS[64], rq[64], rk[64], gC
constexpr int SCR = 2 * BUF;            // wave 2: four diagonal 16x16 blocks
constexpr int SCR_STRIDE = 16 * 20 + 16;
constexpr int NGF = 9;                        // per-token factor arrays per helper
constexpr int GA = SCR + 4 * SCR_STRIDE * 4;  // wave 2 and wave 3 factor arrays
constexpr int LDS_BYTES = GA + 2 * NGF * CH * 4;
static_assert(LDS_BYTES + 3 * KTILE <= 160 * 1024, "LDS budget");
static_assert(B_PF % 16 == 0 && B_VT % 16 == 0 && BUF % 16 == 0, "LDS alignment");

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
    // sequence segments (the segmented launch only)
    int nseg;     // segments per head
    long cps;     // chunks per segment
    float* qh;    // [B*H][T][DK]: outputs of the identity-start columns
    float* nst;   // [B*H][nseg][DK][dv]: segment end states of the value columns
    float* phi;   // [B*H][nseg][DK][DK]: segment transitions (identity-start end states)
};

// ---------------------------------------------------------------------------
// layouts
// ---------------------------------------------------------------------------

// Byte offset of term `plane` (0 = hi, 1 = lo) for `lane` in the fragment of
// (block row R, k-step t), t <= R / 2.
__device__ __forceinline__ int frag_off(int R, int t, int plane, int lane) {
    const int f = (R < 2) ? R : 2 + 2 * (R - 2) + t;
    return ((f * 2 + plane) * 64 + lane) * 16;
}

__device__ __forceinline__ int f32_off(int s, int plane, int lane) { return ((s * 2 + plane) * 64 + lane) * 16; }
__device__ __forceinline__ int f16_off(int s, int plane, int lane) {
    return TF16 + ((s * 2 + plane) * 64 + lane) * 8;
}

// ---------------------------------------------------------------------------
// helper-wave pieces
// ---------------------------------------------------------------------------

// Rows of a chunk in MFMA operand layout: lane (ln, g) holds, for row block
// R and k-step t, the 8 channels 32t + 8g .. +7 of token 16R + ln.
struct RowOps {
    uint4 d[4][4];  // [R][t]
};

// Registers each helper wave carries from one chunk to the next.
struct Wave2Regs {
    float la, be;   // this lane's token gates
};
struct Wave3Regs {
    RowOps q;       // query rows
    uint4 v[4];     // tokens 4q + i (q = lane % 16), value columns 8m .. 8m + 7 (m = lane / 16)
    float gam1;     // this lane's scalar value gain
    float la, be;   // this lane's token gates
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

// Stage operand rows into a swizzled LDS tile (one 16-byte chunk per row and k-step).
__device__ __forceinline__ void stage_rows(const RowOps& ops, uint16_t* tile, int ln, int g) {
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            *reinterpret_cast<uint4*>(tile + kq_off(16 * R + ln, 32 * tt + 8 * g)) = ops.d[R][tt];
}

// Write one operand fragment (8 values of this lane) as hi/lo bf16 terms.
__device__ __forceinline__ void put_frag(char* base, int R, int t, int lane, const f32x4& lo4,
                                         const f32x4& hi4) {
    bf16x8 h[2];
    split_pair(lo4, hi4, h);
    *reinterpret_cast<bf16x8*>(base + frag_off(R, t, 0, lane)) = h[0];
    *reinterpret_cast<bf16x8*>(base + frag_off(R, t, 1, lane)) = h[1];
}

__device__ __forceinline__ void put_f32(char* base, int s, int lane, const f32x4& lo4, const f32x4& hi4) {
    bf16x8 h[2];
    split_pair(lo4, hi4, h);
    *reinterpret_cast<bf16x8*>(base + f32_off(s, 0, lane)) = h[0];
    *reinterpret_cast<bf16x8*>(base + f32_off(s, 1, lane)) = h[1];
}
__device__ __forceinline__ void put_f16(char* base, int s, int lane, const f32x4& v) {
    bf16x4 h[2];
    split_d(v, h);
    *reinterpret_cast<bf16x4*>(base + f16_off(s, 0, lane)) = h[0];
    *reinterpret_cast<bf16x4*>(base + f16_off(s, 1, lane)) = h[1];
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// SEG: the segmented launch (a chunk range per workgroup, identity-start
// columns, segment end states); a separate instantiation so that the one-pass
// kernel carries none of it.
template <bool SEG>
__global__ void __launch_bounds__(NTHR) chunk_fact_kernel(FactParams p) {
    // Key tiles: a ring of three slots, chunk c in slot c % 3.  The slots are
    // separate LDS objects so that the compiler can tell the slot being filled
    // by DMA from the slot being read (a compile-time choice in wave 2's loop)
    // and does not make the reads wait for the DMA.
    __shared__ __attribute__((aligned(16))) uint16_t ks0[CH * DK];
    __shared__ __attribute__((aligned(16))) uint16_t ks1[CH * DK];
    __shared__ __attribute__((aligned(16))) uint16_t ks2[CH * DK];
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
    auto ktile = [&](long c) -> uint16_t* {
        const unsigned m = static_cast<unsigned>(c) % 3u;
        return m == 0 ? ks0 : (m == 1 ? ks1 : ks2);
    };
    // slot S as an LDS-typed pointer (S known at compile time)
    auto kslot = [&](auto slot) -> lds_u16* {
        constexpr int S = decltype(slot)::value;
        if constexpr (S == 0) return (lds_u16*)(ks0);
        else if constexpr (S == 1) return (lds_u16*)(ks1);
        else return (lds_u16*)(ks2);
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int ln = lane & 15;
    const int ntile = p.dv / DVT;
    // Workgroups are dealt round-robin to the XCDs; when the head count allows,
    // give all workgroups of a head the same XCD so they share its L2 for the
    // key, query and gate reads.  The segmented launch has, per head, segment
    // 0's value tiles, then for each later segment its value tiles and the
    // DK / DVT identity tiles.
    const int units = SEG ? ntile + (p.nseg - 1) * (ntile + DK / DVT) : ntile;
    const long nbh = gridDim.x / units;
    long bh;
    int u;
    if (nbh % kXcds == 0) {
        const long slot = blockIdx.x / kXcds;
        u = static_cast<int>(slot % units);
        bh = (slot / units) * kXcds + blockIdx.x % kXcds;
    } else {
        bh = blockIdx.x / units;
        u = static_cast<int>(blockIdx.x % units);
    }
    int tile = u, seg = 0;
    bool ident = false;  // identity-start columns (key channels j0 .. j0 + 31)
    if (SEG && u >= ntile) {
        const int per_seg = ntile + DK / DVT;
        seg = 1 + (u - ntile) / per_seg;
        const int r = (u - ntile) % per_seg;
        ident = r >= ntile;
        tile = ident ? r - ntile : r;
    }
    const int j0 = tile * DVT;
    // value columns this workgroup reads (identity-start columns read none; 0
    // keeps their address arithmetic inside the value and gain rows)
    const int jv = (SEG && ident) ? 0 : j0;
    // this workgroup's chunks: [c0, c0 + nchunks); chunk indices below are
    // relative to c0 (key slots and buffers follow them), tokens start at tb
    const long ntot = (p.T + CH - 1) / CH;
    const long c0 = SEG ? seg * p.cps : 0;
    const long nchunks = SEG ? max(0L, min(p.cps, ntot - c0)) : ntot;
    const long tb = c0 * CH;

    if (wave < NCHAIN) {
        // =========================== chain waves ===========================
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
                for (int e = 0; e < 4; ++e)
                    sacc[ib][e] = p.S0[(bh * DK + srow(ib, g, e)) * p.dv + col];
        } else {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) sacc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // o of chunk c is stored during chunk c + 1, after its Y products are
        // issued: the stores can then wait for the memory pipe (shared with the
        // helpers' key DMA and loads) while the MFMAs run
        f32x4 opend[4];
        auto store_o = [&](long cc) {
            const int c4 = j0 + 16 * wave + 4 * g;
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const long tok = tb + cc * CH + 16 * R + ln;
                if (tok >= p.T) continue;
                if (SEG && ident) {
                    // Phi_t^T q_t: the output of the identity-start columns
                    *reinterpret_cast<f32x4*>(p.qh + (bh * p.T + tok) * DK + c4) = opend[R];
                    continue;
                }
                const long oi = (bh * p.T + tok) * p.dv + c4;
                if (p.o_bf16) {
                    uint2 pk;
                    pk.x = f32_to_bf16_bits(opend[R][0]) | (static_cast<uint32_t>(f32_to_bf16_bits(opend[R][1])) << 16);
                    pk.y = f32_to_bf16_bits(opend[R][2]) | (static_cast<uint32_t>(f32_to_bf16_bits(opend[R][3])) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + oi) = pk;
                } else {
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + oi) = opend[R];
                }
            }
        };
        // Key rows of a chunk as Y's A operands, and the state as x32 B operands
        // (k = key channel).  The key tile of chunk c + 1 is in LDS while chunk
        // c is processed (it is fetched two chunks ahead), so both are prepared
        // at the end of chunk c, before the barrier the chain would otherwise
        // wait at, and chunk c + 1 starts with its Y products.
        bf16x8 ka[4][4], bS[4][2];
        auto prep_next = [&](long cn) {
            const uint16_t* sK = ktile(cn);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    ka[t][b] = *reinterpret_cast<const bf16x8*>(sK + kq_off(16 * b + ln, 32 * t + 8 * g));
#pragma unroll
            for (int t = 0; t < 4; ++t) split_pair(sacc[2 * t], sacc[2 * t + 1], bS[t]);
        };
        __syncthreads();  // the helpers have staged the first key tile
        if (nchunks > 0) prep_next(0);
        __syncthreads();  // ... and prepared chunk 0
        for (long c = 0; c < nchunks; ++c) {
            const char* cur = smem + (c & 1) * BUF;
            const uint16_t* sK = ktile(c);
            const uint16_t* sQ = reinterpret_cast<const uint16_t*>(cur + B_Q);
            const float* sc = reinterpret_cast<const float*>(cur + B_SC);
            const float* sVt = reinterpret_cast<const float*>(cur + B_VT) + (16 * wave + ln) * VTS;
            // Y = K S and Z = Q S with raw bf16 rows as A operands.  The four row
            // blocks are independent accumulation chains; each k-step issues one
            // MFMA per block so consecutive MFMAs never wait on each other.
            f32x4 y[4], z[4];
            auto rows_x_state = [&](const uint16_t* tile, bool transposed, int t, f32x4 (&acc)[4]) {
                bf16x8 a[4];
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    a[b] = *reinterpret_cast<const bf16x8*>(tile + kq_off(16 * b + ln, 32 * t + 8 * g));
                if (!transposed) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc[b] = mfma32(a[b], bS[t][1], acc[b]);
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc[b] = mfma32(a[b], bS[t][0], acc[b]);
                } else {
                    // operands swapped: the result is the transposed block, lane (ln, g)
                    // holding row 16b + ln, value columns 4g .. 4g + 3
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc[b] = mfma32(bS[t][1], a[b], acc[b]);
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc[b] = mfma32(bS[t][0], a[b], acc[b]);
                }
            };
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                y[a] = f32x4{0.f, 0.f, 0.f, 0.f};
                z[a] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int b = 0; b < 4; ++b) y[b] = mfma32(ka[t][b], bS[t][1], y[b]);
#pragma unroll
                for (int b = 0; b < 4; ++b) y[b] = mfma32(ka[t][b], bS[t][0], y[b]);
            }
            if (c > 0) store_o(c - 1);
            // X = Vt - diag(sb Gamma) Y
            f32x4 x[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 rs = *reinterpret_cast<const f32x4*>(sc + 16 * a + 4 * g);
                const f32x4 vv = *reinterpret_cast<const f32x4*>(sVt + 16 * a + 4 * g);
                x[a] = vv - rs * y[a];
            }
            // U by block forward substitution; the B operands of later steps are
            // the hi/lo splits of the blocks already solved
            const char* tf = cur + B_TF;
            auto a16 = [&](int sl, bf16x4 (&o)[2]) {
                o[0] = *reinterpret_cast<const bf16x4*>(tf + f16_off(sl, 0, lane));
                o[1] = *reinterpret_cast<const bf16x4*>(tf + f16_off(sl, 1, lane));
            };
            auto a32 = [&](int sl, bf16x8 (&o)[2]) {
                o[0] = *reinterpret_cast<const bf16x8*>(tf + f32_off(sl, 0, lane));
                o[1] = *reinterpret_cast<const bf16x8*>(tf + f32_off(sl, 1, lane));
            };
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 u[4], W[4];
            bf16x4 bu[4][2], a4[2];
            bf16x8 a8[2];
            // W_R = D_R X_R: independent of each other and of U
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                bf16x4 bx[2];
                split_d(x[R], bx);
                a16(F16_D0 + R, a4);
                W[R] = mm22x16(a4, bx, zero);
            }
            u[0] = W[0];
            split_d(u[0], bu[0]);
            a16(F16_N10, a4);
            u[1] = mm22x16(a4, bu[0], W[1]);
            split_d(u[1], bu[1]);
            bf16x8 bU[2][2];
            bU[0][0] = cat4(bu[0][0], bu[1][0]);
            bU[0][1] = cat4(bu[0][1], bu[1][1]);
            a32(F32_N2, a8);
            u[2] = mm22(a8, bU[0], W[2]);
            a32(F32_N3, a8);
            f32x4 w3 = mm22(a8, bU[0], W[3]);
            split_d(u[2], bu[2]);
            a16(F16_N32, a4);
            u[3] = mm22x16(a4, bu[2], w3);
            split_d(u[3], bu[3]);
            bU[1][0] = cat4(bu[2][0], bu[3][0]);
            bU[1][1] = cat4(bu[2][1], bu[3][1]);

            // S <- Gamma_63 S + K^T diag(sb exp(G_63 - G)) U  (first: it feeds the next chunk)
            f32x4 us[4];
#pragma unroll
            for (int R = 0; R < 4; ++R)
                us[R] = u[R] * *reinterpret_cast<const f32x4*>(sc + 2 * CH + 16 * R + 4 * g);
            bf16x8 bUs[2][2];
            split_pair(us[0], us[1], bUs[0]);
            split_pair(us[2], us[3], bUs[1]);
            const float gC = sc[3 * CH];
#pragma unroll
            for (int ib = 0; ib < 8; ++ib) sacc[ib] *= gC;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // A operand: K^T rows srow(ib, .) (channels), k-slots = tokens
                // {32t + 4g + 0..3, 32t + 16 + 4g + 0..3}, via transpose reads: lane
                // ln of each 16 points at token 32t + 4g + ln / 4 and the 4 channels
                // 32 (ib / 2) + 4 (ib % 2) + 8 (ln % 4) .. + 3.
                bf16x8 ak[8];
                const int tokA = 32 * t + 4 * g + (ln >> 2);
#pragma unroll
                for (int ib = 0; ib < 8; ++ib) {
                    const int pcol = 32 * (ib >> 1) + 4 * (ib & 1) + 8 * (ln & 3);
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(sK + kq_off(tokA, pcol)));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(sK + kq_off(tokA + 16, pcol)));
                    // whole-vector reinterpretation (an element-wise short -> bf16
                    // bit_cast loop is mis-lowered by this compiler: it replicates
                    // element 0)
                    ak[ib] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
                for (int ib = 0; ib < 8; ++ib) sacc[ib] = mfma32(ak[ib], bUs[t][1], sacc[ib]);
#pragma unroll
                for (int ib = 0; ib < 8; ++ib) sacc[ib] = mfma32(ak[ib], bUs[t][0], sacc[ib]);
            }

            // Z = Q S with the state of the chunk start (bS): off the recurrence's
            // critical path, so it is issued after the state update
#pragma unroll
            for (int t = 0; t < 4; ++t) rows_x_state(sQ, true, t, z);

            // O = diag(Gamma) Z + P U, transposed: with U as the A operand and the P
            // fragments as the B operand, lane (ln, g) ends up with row 16R + ln,
            // value columns 4g .. 4g + 3 (the layout z already has), so each row
            // block leaves in one 16-byte store per lane
            const char* pf = cur + B_PF;
            f32x4 oacc[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) oacc[R] = sc[CH + 16 * R + ln] * z[R];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 ap[4][2];
#pragma unroll
                for (int R = 2 * t; R < 4; ++R) {
                    ap[R][0] = *reinterpret_cast<const bf16x8*>(pf + frag_off(R, t, 0, lane));
                    ap[R][1] = *reinterpret_cast<const bf16x8*>(pf + frag_off(R, t, 1, lane));
                }
#pragma unroll
                for (int R = 2 * t; R < 4; ++R) oacc[R] = mfma32(bU[t][0], ap[R][1], oacc[R]);
#pragma unroll
                for (int R = 2 * t; R < 4; ++R) oacc[R] = mfma32(bU[t][1], ap[R][0], oacc[R]);
#pragma unroll
                for (int R = 2 * t; R < 4; ++R) oacc[R] = mfma32(bU[t][0], ap[R][0], oacc[R]);
            }
#pragma unroll
            for (int R = 0; R < 4; ++R) opend[R] = oacc[R];
            if (c + 1 < nchunks) prep_next(c + 1);
            __syncthreads();
        }
        if (nchunks > 0) store_o(nchunks - 1);
        if constexpr (SEG) {
            // the segment's end state: value columns, or the transition
            const long sbase = (bh * p.nseg + seg) * DK;
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (ident) p.phi[(sbase + srow(ib, g, e)) * DK + col] = sacc[ib][e];
                    else p.nst[(sbase + srow(ib, g, e)) * p.dv + col] = sacc[ib][e];
                }
        } else if (p.ST) {
#pragma unroll
            for (int ib = 0; ib < 8; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p.ST[(bh * DK + srow(ib, g, e)) * p.dv + col] = sacc[ib][e];
        }
        return;
    }

    // ============================= helper waves =============================
    const bool w2 = wave == NCHAIN;  // else wave 3

    // Registers: both helpers hold their chunk-c gates while they prepare chunk
    // c, wave 3 also its chunk-c query rows and value tile; wave 2 fetches key
    // tiles into LDS one chunk ahead.  Loads are clamped to row T - 1; rows past T are
    // finite copies that every product below multiplies by a zero gain.
    auto load_gates = [&](long c, float& la, float& be) {
        const long tok = bh * p.T + min(tb + c * CH + lane, p.T - 1);
        la = p.log_alpha[tok];
        be = p.beta[tok];
    };
    // Key tile of chunk c straight from HBM into its LDS slot (LDS DMA, no
    // registers): instruction m fills rows 4m .. 4m + 3, lane i landing at row
    // 4m + i / 16, physical 16-byte chunk i % 16, so it fetches the logical
    // chunk that the tile swizzle puts there.  A buffer resource per head
    // (records = T rows) makes rows past T read as zeros.  The swizzle of row
    // r = 4m + i / 16 is f = 4 (r % 4) + (r / 4) % 4 = 4 (i / 16) + m % 4, so
    // four per-lane offsets cover all m.
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.k + bh * p.T * DK), 0, static_cast<int>(p.T * DK * 2), 0x00020000);
    unsigned koff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        koff[q] = (lane >> 4) * DK * 2 + 16 * ((lane & 15) ^ (((lane >> 4) << 2) | q));
    auto dma_keys = [&](long c, lds_u16* tile) {
        const unsigned cb = static_cast<unsigned>((tb + c * CH) * DK * 2);
#pragma unroll
        for (int m = 0; m < 16; ++m)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(tile + 4 * m * DK), 16,
                                                     cb + m * 4 * DK * 2 + koff[m & 3], 0, 0, 0);
    };
    auto load3 = [&](long c, Wave3Regs& R3) {
        const long t0 = tb + c * CH;
        load_gates(c, R3.la, R3.be);
        load_rows(R3.q, p.q, bh, p.T, t0, ln, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const long tk = bh * p.T + min(t0 + 4 * ln + i, p.T - 1);
            // (unconditional: a load issued on one path only, or a select on the
            // loaded value here, makes the compiler wait for the load at once;
            // the identity-start columns zero their values where they are staged)
            R3.v[i] = *reinterpret_cast<const uint4*>(p.v + tk * p.dv + jv + 8 * g);
        }
        if (!p.gvec) R3.gam1 = p.gsrc[(bh * p.T + min(t0 + lane, p.T - 1)) * p.gts];
    };
    // rows of a staged tile as 16x16x32 operands: block b, k-step t
    auto tile_op = [&](const uint16_t* tile, int b, int t) {
        return *reinterpret_cast<const bf16x8*>(tile + kq_off(16 * b + ln, 32 * t + 8 * g));
    };

    // Per-token gates and decay factors of chunk c.  Lane r holds token r:
    // inclusive cumulative log2 decay G_r (rows past T add nothing) and
    // sb_r = sqrt(beta_r) (0 past T: no erase, no write).  The decay between
    // two tokens of a chunk is split into a row and a column factor, each a
    // power of two of one token's G relative to a reference, so that the
    // Gram blocks need no per-element exponentials:
    //   diagonal block R (reference Gm = G at row 16R + 7, |G_r - Gm| <= 115
    //   by the per-token clamp): FA = [sb_r] 2^(G_r - Gm), FB = sb_s 2^(Gm - G_s);
    //   off-diagonal R > J (reference Ge_J = G at row 16J + 15, both factors
    //   <= 1): FE_J = [sb_r] 2^(G_r - Ge_J), FF = sb_s 2^(Ge_J - G_s) for s in J.
    // Row factors carry sb_r only for T (wave 2), not for P (wave 3).
    // The diagonal-block split needs |G_r - Gm| inside the fp32 range, which a
    // per-token log decay >= kLogAlphaMin guarantees.  A chunk with a stronger
    // decay (a wave-uniform flag) forms its diagonal blocks element by element
    // instead, 2^(G_r - G_s) from the per-token G and sb kept in GL and SBV;
    // log decays are floored at kLogAlphaFloor, where alpha (e^-80) is below
    // what an fp32 state can resolve, so the result is the recurrence's.
    struct GateVals {
        float gl, sb, G2last;
        float fa, ff;  // this lane's FA and FF factors (token = lane)
        bool strong;   // some token of the chunk decays below kLogAlphaMin
    };
    float* gw = reinterpret_cast<float*>(smem + GA) + (w2 ? 0 : NGF * CH);
    enum { FA = 0, FB = CH, FF = 2 * CH, FE = 3 * CH, SG = 6 * CH, GL = 7 * CH, SBV = 8 * CH };
    auto gate_prologue = [&](long c, float la, float be, bool row_sb) {
        GateVals v;
        const bool ok = tb + c * CH + lane < p.T;
        const float lac = (p.has_alpha && ok) ? fmaxf(la, kLogAlphaFloor) : 0.0f;
        v.strong = __builtin_amdgcn_ballot_w64(lac < kLogAlphaMin) != 0;
        v.gl = wave_incl_scan(lac * kLog2e);
        v.sb = ok ? sqrt_hw(be) : 0.0f;
        auto at = [&](int r) {
            return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v.gl), r));
        };
        v.G2last = at(63);
        const float ge0 = at(15), ge1 = at(31), ge2 = at(47);
        const float gm0 = at(7), gm1 = at(23), gm2 = at(39), gm3 = at(55);
        const int R = lane >> 4;
        const float gm = R == 0 ? gm0 : (R == 1 ? gm1 : (R == 2 ? gm2 : gm3));
        const float geR = R == 0 ? ge0 : (R == 1 ? ge1 : ge2);  // unused for R == 3
        const float rs = row_sb ? v.sb : 1.0f;
        v.fa = rs * ex2(v.gl - gm);
        v.ff = v.sb * ex2(fminf(geR - v.gl, 0.0f));
        gw[FA + lane] = v.fa;
        gw[FB + lane] = v.sb * ex2(gm - v.gl);
        gw[FF + lane] = v.ff;
        gw[FE + lane] = rs * ex2(fminf(v.gl - ge0, 0.0f));
        gw[FE + CH + lane] = rs * ex2(fminf(v.gl - ge1, 0.0f));
        gw[FE + 2 * CH + lane] = rs * ex2(fminf(v.gl - ge2, 0.0f));
        gw[GL + lane] = v.gl;
        gw[SBV + lane] = v.sb;
        return v;
    };

    // Everything chunk c needs goes into `buf`; wave 2 additionally fetches the
    // key tile of chunk c + 1.
    auto prepare2 = [&](long c, char* buf, Wave2Regs& R2, auto slot) {
        const float la = R2.la, be = R2.be;
        const GateVals gv = gate_prologue(c, la, be, true);
        // ---- wave 2: fetch the next key tile, form T, invert the diagonal blocks ----
        // (unconditional: past the last chunk it refetches row T - 1 into a slot
        // that nothing reads any more, which keeps the destination a constant)
        constexpr int S = decltype(slot)::value;
        dma_keys(c + 1, kslot(std::integral_constant<int, (S + 1) % 3>{}));
        // unconditional as well (the token index is clamped): a load issued on
        // one path only makes the compiler drain every outstanding load,
        // including the key DMA just issued, before the next LDS read
        load_gates(c + 1, R2.la, R2.be);
        const uint16_t* kt = (const uint16_t*)kslot(slot);
        f32x4 tr[4][4];
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int J = 0; J <= R; ++J) tr[R][J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 kr[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) kr[b] = tile_op(kt, b, t);
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                // diagonal blocks as row segments (lane (ln, g): row ln, columns
                // 4g + e), off-diagonal blocks in accumulator layout of T_RJ
                tr[R][R] = mfma32(kr[R], kr[R], tr[R][R]);
#pragma unroll
                for (int J = 0; J < R; ++J) tr[R][J] = mfma32(kr[R], kr[J], tr[R][J]);
            }
        }
        float* scr = reinterpret_cast<float*>(smem + SCR);
        // tc[R][J] holds T[16R + 4g + e][16J + ln] for J < R (T_RJ in accumulator
        // layout); diagonal blocks (row ln, columns 4g + e) go to the scratch
        // negated, as the solve consumes them (a negation folded into the solve's
        // FMAs would keep them from taking the row broadcast as a DPP operand).
        f32x4 tc[4][4];
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int J = 0; J <= R; ++J) {
                f32x4 acc = tr[R][J];
                // per-row scalars by lane permute, not from LDS: this wave has
                // just issued the next key DMA, and the compiler would make an
                // LDS read it cannot tell apart from that DMA wait for all of it
                if (J == R) {
                    if (!gv.strong) {
                        const f32x4 cf = *reinterpret_cast<const f32x4*>(gw + FB + 16 * R + 4 * g);
                        const float rf = lane_get(gv.fa, 16 * R + ln);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[e] = (4 * g + e < ln) ? -(acc[e] * rf * cf[e]) : 0.0f;
                    } else {
                        const f32x4 gs = *reinterpret_cast<const f32x4*>(gw + GL + 16 * R + 4 * g);
                        const f32x4 bs = *reinterpret_cast<const f32x4*>(gw + SBV + 16 * R + 4 * g);
                        const float gr = lane_get(gv.gl, 16 * R + ln);
                        const float br = lane_get(gv.sb, 16 * R + ln);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[e] = (4 * g + e < ln) ? -(acc[e] * br * bs[e] * ex2(gr - gs[e])) : 0.0f;
                    }
                    *reinterpret_cast<f32x4*>(scr + R * SCR_STRIDE + ln * 20 + 4 * g) = acc;
                } else {
                    const f32x4 rf = *reinterpret_cast<const f32x4*>(gw + FE + J * CH + 16 * R + 4 * g);
                    tc[R][J] = acc * rf * lane_get(gv.ff, 16 * J + ln);
                }
            }
        // diagonal blocks: D_R = (I + T_RR)^-1 row by row, one row per lane
        // (lane = (R, row r); a DPP row of 16 lanes is one block).  Once row j
        // is final it is broadcast across its block and every row r takes
        // x_r -= T_rj x_j; rows r <= j have T_rj = 0 and stay unchanged, and
        // x_j is zero beyond column j, so step j touches columns 0..j only.
        // D_R overwrites -T_RR in the scratch (row-major, row stride 20).
        {
            float* Brow = scr + (lane >> 4) * SCR_STRIDE + (lane & 15) * 20;
            float ntr[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(Brow + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) ntr[4 * q + e] = v[e];
            }
            float x[16];
#pragma unroll
            for (int cc = 0; cc < 16; ++cc) x[cc] = (cc == (lane & 15)) ? 1.0f : 0.0f;
            block_row_solve(x, ntr);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f32x4*>(Brow + 4 * q) = f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
        }
        // N_RJ = D_R T_RJ.  With tc = T_RJ and drow(R) = D_R^T in accumulator
        // layout, an MFMA with the T block as the A operand (a register block
        // used as A acts as its transpose) gives (D_R T_RJ)^T in accumulator
        // layout: lane (ln, g) holds row ln, columns 4g .. 4g + 3 of N_RJ,
        // which is its A-operand fragment.  The same holds for drow(R) and D_R.
        char* tf = buf + B_TF;
        bf16x4 bd[4][2];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            split_d(*reinterpret_cast<const f32x4*>(scr + R * SCR_STRIDE + ln * 20 + 4 * g), bd[R]);
            *reinterpret_cast<bf16x4*>(tf + f16_off(F16_D0 + R, 0, lane)) = bd[R][0];
            *reinterpret_cast<bf16x4*>(tf + f16_off(F16_D0 + R, 1, lane)) = bd[R][1];
        }
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 nb[4][4];
#pragma unroll
        for (int R = 1; R < 4; ++R)
#pragma unroll
            for (int J = 0; J < R; ++J) {
                bf16x4 bt[2];
                split_d(-tc[R][J], bt);
                nb[R][J] = mm22x16(bt, bd[R], zero);
            }
        put_f16(tf, F16_N10, lane, nb[1][0]);
        put_f16(tf, F16_N32, lane, nb[3][2]);
        put_f32(tf, F32_N2, lane, nb[2][0], nb[2][1]);
        put_f32(tf, F32_N3, lane, nb[3][0], nb[3][1]);
    };
    auto prepare3 = [&](long c, char* buf, Wave3Regs& R3) {
        const float la = R3.la, be = R3.be;
        const long t0 = tb + c * CH;
        const GateVals gv = gate_prologue(c, la, be, false);
        // ---- wave 3: form P, stage Q, V (transposed), row scales ----
        // raw query-key products (keys from the staged tile) first, so the
        // registers can be refilled
        const uint16_t* kt = ktile(c);
        f32x4 pb[4][4];
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int S = 0; S <= R; ++S) pb[R][S] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 kr[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) kr[b] = tile_op(kt, b, t);
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int S = 0; S <= R; ++S) pb[R][S] = mfma32(kr[S], as_bf16x8(R3.q.d[R][t]), pb[R][S]);
        }
        stage_rows(R3.q, reinterpret_cast<uint16_t*>(buf + B_Q), ln, g);
        float* sc = reinterpret_cast<float*>(buf + B_SC);
        const float eg = ex2(gv.gl);
        sc[lane] = gv.sb * eg;                      // rows of K.Gamma
        sc[CH + lane] = eg;                         // rows of Q.Gamma
        sc[2 * CH + lane] = gv.sb * ex2(gv.G2last - gv.gl);  // rows of Khat
        if (lane == 0) sc[3 * CH] = ex2(gv.G2last);          // chunk decay
        // value tile, transposed and scaled by sqrt(gamma): lane (q = ln, m = g)
        // holds tokens 4q .. 4q + 3 of columns 8m .. 8m + 7, one 16-byte write
        // per column; rows past T get 0
        float* sVt = reinterpret_cast<float*>(buf + B_VT);
        f32x4 sg4[8];
        if (!p.gvec) {
            gw[SG + lane] = (tb + c * CH + lane < p.T) ? sqrt_hw(R3.gam1) : 0.0f;
            const f32x4 s4 = *reinterpret_cast<const f32x4*>(gw + SG + 4 * ln);
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) sg4[cc] = s4;
        } else {
            // all 32 gains loaded (rows past T reread the last row) before the
            // mask: a load behind the row test would wait for each in turn
            float gr[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float* src = p.gsrc + (bh * p.T + min(t0 + 4 * ln + i, p.T - 1)) * p.gts + jv + 8 * g;
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) gr[i][cc] = src[cc];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float m = t0 + 4 * ln + i < p.T ? 1.0f : 0.0f;
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) sg4[cc][i] = sqrt_hw(gr[i][cc]) * m;
            }
        }
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            f32x4 col4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                col4[i] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(&R3.v[i])[cc]);
            // identity-start columns run with zero values (j0 indexes key channels)
            const f32x4 val = (SEG && ident) ? f32x4{0.f, 0.f, 0.f, 0.f} : sg4[cc] * col4;
            *reinterpret_cast<f32x4*>(sVt + (8 * g + cc) * VTS + 4 * ln) = val;
        }
        if (c + 1 < nchunks) load3(c + 1, R3);
        // P^T blocks: pb[R][S] holds P[16R + ln][16S + 4g + e]
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int S = 0; S <= R; ++S) {
                if (S == R) {
                    if (!gv.strong) {
                        const f32x4 cf = *reinterpret_cast<const f32x4*>(gw + FB + 16 * R + 4 * g);
                        const float rf = gw[FA + 16 * R + ln];
#pragma unroll
                        for (int e = 0; e < 4; ++e) pb[R][S][e] = (4 * g + e <= ln) ? pb[R][S][e] * rf * cf[e] : 0.0f;
                    } else {
                        const f32x4 gs = *reinterpret_cast<const f32x4*>(gw + GL + 16 * R + 4 * g);
                        const f32x4 bs = *reinterpret_cast<const f32x4*>(gw + SBV + 16 * R + 4 * g);
                        const float gr = gw[GL + 16 * R + ln];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pb[R][S][e] = (4 * g + e <= ln) ? pb[R][S][e] * bs[e] * ex2(gr - gs[e]) : 0.0f;
                    }
                } else {
                    const f32x4 cf = *reinterpret_cast<const f32x4*>(gw + FF + 16 * S + 4 * g);
                    pb[R][S] = pb[R][S] * (gw[FE + S * CH + 16 * R + ln] * cf);
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
    };

    // Prologue: wave 2 fetches the first key tile; both helpers hold the gates
    // (wave 3 also the queries and values) of chunk 0.  prepare(c) refills the registers as soon as they
    // have been consumed, which leaves a whole chunk period for loads to land.
    // The two waves run separate copies of the loop (same barrier sequence) so
    // that each keeps only its own registers live.
    if (w2) {
        Wave2Regs R2;
        if (nchunks > 0) {
            dma_keys(0, kslot(std::integral_constant<int, 0>{}));
            load_gates(0, R2.la, R2.be);
        }
        __syncthreads();
        if (nchunks > 0) prepare2(0, smem, R2, std::integral_constant<int, 0>{});
        __syncthreads();
        // unrolled by three so that every key slot index is a compile-time
        // constant; one barrier per chunk as in the other waves
        for (long c = 0; c < nchunks; c += 3) {
            if (c + 1 < nchunks) prepare2(c + 1, smem + ((c + 1) & 1) * BUF, R2, std::integral_constant<int, 1>{});
            __syncthreads();
            if (c + 1 < nchunks) {
                if (c + 2 < nchunks) prepare2(c + 2, smem + ((c + 2) & 1) * BUF, R2, std::integral_constant<int, 2>{});
                __syncthreads();
            }
            if (c + 2 < nchunks) {
                if (c + 3 < nchunks) prepare2(c + 3, smem + ((c + 3) & 1) * BUF, R2, std::integral_constant<int, 0>{});
                __syncthreads();
            }
        }
    } else {
        Wave3Regs R3;
        if (nchunks > 0) load3(0, R3);
        __syncthreads();
        if (nchunks > 0) prepare3(0, smem, R3);
        __syncthreads();
        for (long c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) prepare3(c + 1, smem + ((c + 1) & 1) * BUF, R3);
            __syncthreads();
        }
    }
}

}  // namespace

bool chunk_fact_supported(const pdn_chunk_fwd_args& a) {
    // key rows of one head are addressed with 32-bit byte offsets
    return a.qkv_dtype == PDN_BF16 && a.dk == DK && a.dv % DVT == 0 &&
           static_cast<long>(a.T) * DK * 2 <= 0x7fffffffL &&
           a.alpha_mode != PDN_ALPHA_VEC && a.beta_mode == PDN_GATE_SCALAR &&
           a.precond_eps < 0.0f && a.key_mode == PDN_KEY_SYMMETRIC;
}

namespace {

// Sequence segments for few heads and long sequences (fp32 output; the
// correction adds to the stored outputs): as many segments as keep every
// workgroup of the launch resident at once (one per CU, the MI355X count as a
// constant: the segment count sets the workspace size, which a caller may ask
// for before any device is current), at least 8 chunks each, at most 8.
constexpr long kFactSlots = 256;
int fact_segments(const pdn_chunk_fwd_args& a) {
    if (a.o_dtype != PDN_F32) return 1;
    const long nbh = static_cast<long>(a.B) * a.H;
    const long nc = (static_cast<long>(a.T) + CH - 1) / CH;
    const long vt = a.dv / DVT, it = DK / DVT;
    int G = 1;
    for (int g = 2; g <= 8; ++g) {
        if (nc < 8L * g || nbh * (vt * g + it * (g - 1)) > kFactSlots) break;
        G = g;
    }
    return G;
}

// workspace of a segmented launch: Phi_t^T q_t rows [B*H][T][DK], then the
// segment end states [B*H][G][DK][dv], transitions [B*H][G][DK][DK] and start
// states [B*H][G][DK][dv] (fp32)
struct FactSegBufs {
    size_t qh, nst, phi, sst, end;
};
FactSegBufs fact_seg_layout(const pdn_chunk_fwd_args& a, int G) {
    const size_t nbh = static_cast<size_t>(a.B) * a.H;
    FactSegBufs b;
    b.qh = 0;
    b.nst = b.qh + (G > 1 ? nbh * a.T * DK * sizeof(float) : 0);
    b.phi = b.nst + (G > 1 ? nbh * G * DK * a.dv * sizeof(float) : 0);
    b.sst = b.phi + (G > 1 ? nbh * G * DK * DK * sizeof(float) : 0);
    b.end = b.sst + (G > 1 ? nbh * G * DK * a.dv * sizeof(float) : 0);
    return b;
}

}  // namespace

size_t chunk_fact_workspace_bytes(const pdn_chunk_fwd_args& a) {
    return fact_seg_layout(a, fact_segments(a)).end;
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
    const long nbh = static_cast<long>(a.B) * a.H;
    const int G = fact_segments(a);
    const long vt = a.dv / DVT, it = DK / DVT;
    if (G == 1) {
        p.nseg = 1;
        p.cps = 0;
        p.qh = p.nst = p.phi = nullptr;
        chunk_fact_kernel<false><<<dim3(static_cast<unsigned>(nbh * vt)), dim3(NTHR), 0, stream>>>(p);
        return hipGetLastError();
    }
    const long nc = (static_cast<long>(a.T) + CH - 1) / CH;
    char* ws = static_cast<char*>(a.workspace);
    const FactSegBufs sb = fact_seg_layout(a, G);
    p.nseg = G;
    p.cps = (nc + G - 1) / G;
    p.qh = reinterpret_cast<float*>(ws + sb.qh);
    p.nst = reinterpret_cast<float*>(ws + sb.nst);
    p.phi = reinterpret_cast<float*>(ws + sb.phi);
    const long nwg = nbh * (vt + (G - 1) * (vt + it));
    chunk_fact_kernel<true><<<dim3(static_cast<unsigned>(nwg)), dim3(NTHR), 0, stream>>>(p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_seg_finish(p.nst, p.phi, reinterpret_cast<float*>(ws + sb.sst), a.ST, p.qh,
                             static_cast<float*>(a.o), nbh, a.T, G, p.cps * CH, a.dv, stream);
}

}  // namespace pdn
