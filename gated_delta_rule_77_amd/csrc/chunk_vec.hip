// Per-channel-gate prefill: the preconditioner pre-pass, the sequence-segment
// kernels and the host side (workspace layout and launch sequence).  The
// preparation and chain kernels are in chunk_vec.h.
#include "chunk_vec.h"

namespace pdn {
namespace {

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
    if constexpr (AVEC && BVEC && !STAB) {
        if (km == PDN_KEY_SYMMETRIC) {
            launch_vec_prep_sym_vec<PRE>(pp, static_cast<unsigned>(nblk), stream);
            return;
        }
    }
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
