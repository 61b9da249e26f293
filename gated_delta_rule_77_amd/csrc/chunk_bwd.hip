// Backward of the chunked gated delta rule: host side (workspace layout and
// launch sequence) and the kernels built with the default scheduler.  The
// kernels themselves are in chunk_bwd.h.
#include "chunk_bwd.h"

namespace pdn {
namespace {

// T == 0: dS0 = dST (or 0), dA0 = 0
__global__ void bwd_copy_kernel(float* dst, const float* src, long n) {
    const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct BwdLayout {
    size_t rec, st, dst, U, Z, dgr, apre, ksum, dAin, dAc, dAsuf, mu, end;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

BwdLayout bwd_layout(const pdn_chunk_bwd_args& a) {
    const pdn_chunk_fwd_args& f = a.fwd;
    const size_t nbh = static_cast<size_t>(f.B) * f.H;
    const size_t nc = (static_cast<size_t>(f.T) + BC - 1) / BC;
    const size_t dk = f.dk, dv = f.dv;
    const size_t recf = 3 * BC * dk + 2 * BC * BC + dk + BC * dv;
    const size_t dgrf = 3 * BC * dk + dk;
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
    L.mu = take(pre && f.precond_mode == PDN_PRECOND_STABILISED ? nbh * nc * BC : 0);
    L.end = o;
    return L;
}

template <int DK, bool BF16>
hipError_t run_bwd(const pdn_chunk_bwd_args& a, const BwdParams& p, hipStream_t s) {
    const unsigned nbh = static_cast<unsigned>(p.nbh);
    const unsigned nch = static_cast<unsigned>(p.nbh * p.nc);
    // state-pass tiles: 32 value columns, or 16 when that still leaves at
    // least half the CUs without a state-pass workgroup (few heads)
    const bool narrow = 2L * p.nbh * (p.dv / JT) <= device_cu_count() / 2;
    const unsigned ntl = static_cast<unsigned>(p.nbh * (p.dv / (narrow ? 16 : JT)));
    (void)a;
    if (p.pre) {
        bwd_ksum_kernel<DK, BF16><<<nch, DK, 0, s>>>(p);
        bwd_scan_kernel<DK, false><<<nbh * (DK / SCAN_CH), SCAN_SEG * SCAN_CH, 0, s>>>(p.ksum, p.apre, p.A0, nullptr,
                                                                                   p.nc);
    }
    if (p.stab) bwd_prep_kernel<DK, BF16, true><<<nch, NT, 0, s>>>(p);
    else bwd_prep_kernel<DK, BF16, false><<<nch, NT, 0, s>>>(p);
    const unsigned sgrid = 2 * kXcds * ((ntl + kXcds - 1) / kXcds);
    if (narrow) bwd_states_kernel<DK, 16><<<sgrid, NT, 0, s>>>(p, static_cast<long>(ntl));
    else launch_bwd_states_wide<DK>(p, sgrid, static_cast<long>(ntl), s);
    launch_bwd_grads<DK, BF16>(p, nch, s);
    if (p.pre) {
        bwd_scan_kernel<DK, true><<<nbh * (DK / SCAN_CH), SCAN_SEG * SCAN_CH, 0, s>>>(p.dAc, p.dAsuf, nullptr, p.dA0,
                                                                                  p.nc);
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
    p.stab = p.pre && f.precond_mode == PDN_PRECOND_STABILISED;
    p.lnx = p.stab ? logf(f.precond_x) : 0.f;
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
    p.mu = at(L.mu);
    const bool bf = f.qkv_dtype == PDN_BF16;
    if (f.dk == 128) return bf ? run_bwd<128, true>(a, p, stream) : run_bwd<128, false>(a, p, stream);
    return bf ? run_bwd<64, true>(a, p, stream) : run_bwd<64, false>(a, p, stream);
}

}  // namespace pdn
