// Host layer of libpdn.so: the extern "C" entry points declared in pdn.h.
// Every entry point validates its arguments before touching the GPU, maps
// HIP errors to PDN_EHIP, and lets no exception escape.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <atomic>
#include <mutex>

#include "kernels.h"
#include "pdn.h"

namespace {

bool valid_dtype(int32_t d) { return d == PDN_F32 || d == PDN_BF16; }
bool valid_alpha(int32_t m) {
    return m == PDN_ALPHA_NONE || m == PDN_ALPHA_SCALAR || m == PDN_ALPHA_VEC;
}
bool valid_beta(int32_t m) { return m == PDN_GATE_SCALAR || m == PDN_GATE_VEC; }
bool valid_gamma(int32_t m) {
    return m == PDN_GATE_SCALAR || m == PDN_GATE_VEC || m == PDN_GAMMA_SAME_AS_BETA;
}
bool valid_key(int32_t m) {
    return m == PDN_KEY_SYMMETRIC || m == PDN_KEY_ERASE_GATE || m == PDN_KEY_WRITE_GATE;
}
// preconditioner mode and bound; x is only read in the stabilised mode
bool valid_precond(float eps, int32_t mode, float x) {
    if (mode != PDN_PRECOND_INVERSE && mode != PDN_PRECOND_STABILISED) return false;
    if (eps >= 0.0f && mode == PDN_PRECOND_STABILISED && !(x > 1.0f && x <= 2.0f)) return false;
    return true;
}

// Largest B*H (and B*H*T) the launch grids and 32/64-bit index math accept.
constexpr long kMaxBH = 1L << 24;
// B * H * T: keeps every launch grid (at most one wave per 32-token chunk and
// (b, h), four per workgroup) below 2^31 workgroups
constexpr long kMaxTokens = 1L << 36;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Gate enums and pointers.  With no tokens to process (need_data false) the
// gate pointers may be NULL.
int check_gates(int32_t amode, const float* la, int32_t bmode, const float* beta,
                int32_t gmode, const float* gamma, float eps, int dk, int dv, bool need_data) {
    if (!valid_alpha(amode) || !valid_beta(bmode) || !valid_gamma(gmode)) return PDN_EINVAL;
    if (need_data) {
        if (amode != PDN_ALPHA_NONE && !la) return PDN_EINVAL;
        if (!beta) return PDN_EINVAL;
        if (gmode != PDN_GAMMA_SAME_AS_BETA && !gamma) return PDN_EINVAL;
    }
    if (gmode == PDN_GAMMA_SAME_AS_BETA && bmode == PDN_GATE_VEC && dk != dv)
        return PDN_EINVAL;
    if (std::isnan(eps)) return PDN_EINVAL;
    return PDN_OK;
}

// check_ws false: everything but the workspace (the size query, made before
// the caller has one)
int check_chunk(const pdn_chunk_fwd_args* a, bool check_ws = true) {
    if (!a) return PDN_EINVAL;
    if (a->B < 1 || a->H < 1 || a->T < 0 || a->dk < 1 || a->dv < 1) return PDN_EINVAL;
    if (!valid_dtype(a->qkv_dtype) || !valid_dtype(a->o_dtype)) return PDN_EINVAL;
    if (static_cast<long>(a->B) * a->H > kMaxBH) return PDN_EUNSUPPORTED;
    if (static_cast<long>(a->B) * a->H * a->T > kMaxTokens) return PDN_EUNSUPPORTED;
    int rc = check_gates(a->alpha_mode, a->log_alpha, a->beta_mode, a->beta, a->gamma_mode,
                         a->gamma, a->precond_eps, a->dk, a->dv, a->T > 0);
    if (rc != PDN_OK) return rc;
    if (!valid_key(a->key_mode)) return PDN_EINVAL;
    if (!valid_precond(a->precond_eps, a->precond_mode, a->precond_x)) return PDN_EINVAL;
    if (a->T > 0 && (!a->q || !a->k || !a->v || !a->o)) return PDN_EINVAL;
    // the kernels use 16-byte vector loads and stores
    const void* ptrs[] = {a->q, a->k, a->v, a->o, a->log_alpha, a->beta, a->gamma,
                          a->precond_A0, a->precond_AT, a->S0, a->ST,
                          check_ws ? a->workspace : nullptr};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return PDN_EINVAL;
    if (a->dk != 64 && a->dk != 128) return PDN_EUNSUPPORTED;
    if (a->dv % 16 != 0 || a->dv > 256) return PDN_EUNSUPPORTED;
    const bool vec = a->alpha_mode == PDN_ALPHA_VEC || a->beta_mode == PDN_GATE_VEC ||
                     a->precond_eps >= 0.0f;
    if (vec && a->dv % 32 != 0) return PDN_EUNSUPPORTED;
    // asymmetric keys and the stabilised preconditioner run on the bf16,
    // dk = 128 per-channel-gate kernels only
    const bool stabilised = a->precond_eps >= 0.0f && a->precond_mode == PDN_PRECOND_STABILISED;
    if ((a->key_mode != PDN_KEY_SYMMETRIC || stabilised) &&
        (a->qkv_dtype != PDN_BF16 || a->dk != 128 || a->dv % 32 != 0))
        return PDN_EUNSUPPORTED;
    if (a->S0 && a->ST && a->S0 != a->ST) {
        // distinct state buffers must not overlap
        const long n = static_cast<long>(a->B) * a->H * a->dk * a->dv;
        const float* s0 = a->S0;
        const float* st = a->ST;
        if (s0 < st + n && st < s0 + n) return PDN_EINVAL;
    }
    if (!check_ws) return PDN_OK;
    const size_t need = pdn::chunk_fwd_workspace_bytes(*a);
    if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return PDN_EWORKSPACE;
    return PDN_OK;
}

// B * H * T for the backward: its per-chunk grids stay below 2^31 workgroups
constexpr long kMaxBwdTokens = 1L << 35;

int check_bwd(const pdn_chunk_bwd_args* a, bool check_ws = true) {
    if (!a) return PDN_EINVAL;
    const pdn_chunk_fwd_args& f = a->fwd;
    if (f.B < 1 || f.H < 1 || f.T < 0 || f.dk < 1 || f.dv < 1) return PDN_EINVAL;
    if (!valid_dtype(f.qkv_dtype)) return PDN_EINVAL;
    if (static_cast<long>(f.B) * f.H > kMaxBH) return PDN_EUNSUPPORTED;
    if (static_cast<long>(f.B) * f.H * f.T > kMaxBwdTokens) return PDN_EUNSUPPORTED;
    const bool data = f.T > 0;
    int rc = check_gates(f.alpha_mode, f.log_alpha, f.beta_mode, f.beta, f.gamma_mode, f.gamma,
                         f.precond_eps, f.dk, f.dv, data);
    if (rc != PDN_OK) return rc;
    if (!valid_key(f.key_mode)) return PDN_EINVAL;
    if (!valid_precond(f.precond_eps, f.precond_mode, f.precond_x)) return PDN_EINVAL;
    if (data) {
        if (!f.q || !f.k || !f.v || !a->dO || !a->dq || !a->dk || !a->dv || !a->dbeta)
            return PDN_EINVAL;
        if (f.alpha_mode != PDN_ALPHA_NONE && !a->dlog_alpha) return PDN_EINVAL;
        if (f.gamma_mode != PDN_GAMMA_SAME_AS_BETA && !a->dgamma) return PDN_EINVAL;
    }
    const void* ptrs[] = {f.q, f.k, f.v, f.log_alpha, f.beta, f.gamma, f.precond_A0, f.S0,
                          a->dO, a->dST, a->dq, a->dk, a->dv, a->dlog_alpha, a->dbeta,
                          a->dgamma, a->dS0, a->dA0, check_ws ? a->workspace : nullptr};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return PDN_EINVAL;
    if (f.dk != 64 && f.dk != 128) return PDN_EUNSUPPORTED;
    if (f.dv % 32 != 0 || f.dv > 256) return PDN_EUNSUPPORTED;
    if (!check_ws) return PDN_OK;
    const size_t need = pdn::chunk_bwd_workspace_bytes(*a);
    if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return PDN_EWORKSPACE;
    return PDN_OK;
}

int check_decode(const pdn_decode_args* a) {
    if (!a) return PDN_EINVAL;
    if (a->B < 1 || a->H < 1 || a->dk < 1 || a->dv < 1) return PDN_EINVAL;
    if (!valid_dtype(a->qkv_dtype) || !valid_dtype(a->o_dtype)) return PDN_EINVAL;
    if (!a->q || !a->k || !a->v || !a->o || !a->S) return PDN_EINVAL;
    int rc = check_gates(a->alpha_mode, a->log_alpha, a->beta_mode, a->beta, a->gamma_mode,
                         a->gamma, a->precond_eps, a->dk, a->dv, true);
    if (rc != PDN_OK) return rc;
    if (!valid_key(a->key_mode)) return PDN_EINVAL;
    if (!valid_precond(a->precond_eps, a->precond_mode, a->precond_x)) return PDN_EINVAL;
    if (a->precond_eps >= 0.0f && !a->precond_A) return PDN_EINVAL;
    if (!aligned16(a->S)) return PDN_EINVAL;  // streamed with 16-byte accesses
    if (static_cast<long>(a->B) * a->H > kMaxBH) return PDN_EUNSUPPORTED;
    if ((a->dk != 64 && a->dk != 128) || (a->dv != 64 && a->dv != 128)) return PDN_EUNSUPPORTED;
    return PDN_OK;
}

// Scratch of pdn_chunk_fwd_noalloc: one copy per GPU, loaded with the code
// object (no allocation call makes it).  In host code `scratch` is a host-side
// stand-in for the symbol, never a device address: every use goes through the
// per-device address from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[PDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept; nullptr if HIP reports an error.
void* scratch_on_current_device() {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

}  // namespace

namespace pdn {

int device_cu_count() {
    // queried once per device (decode launches ask on every step)
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;  // the MI355X count; only grid sizes depend on it
    if (dev < kMaxDevices && (n = cached[dev].load(std::memory_order_relaxed)) > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
    if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace pdn

extern "C" {

int pdn_abi_version(void) { return PDN_ABI_VERSION; }

const char* pdn_strerror(int code) {
    switch (code) {
        case PDN_OK: return "success";
        case PDN_EINVAL: return "invalid argument (null pointer, size or enum value)";
        case PDN_EUNSUPPORTED: return "valid request outside what the kernels support";
        case PDN_EWORKSPACE: return "workspace missing or too small";
        case PDN_EHIP: return "HIP runtime error at launch";
        case PDN_ESCRATCH:
            return "call needs more scratch than pdn_chunk_fwd_noalloc holds "
                   "(PDN_NOALLOC_SCRATCH_BYTES): pass a workspace to pdn_chunk_fwd";
        default: return "unknown error code";
    }
}

int pdn_chunk_fwd_workspace_size(const pdn_chunk_fwd_args* args, size_t* bytes) {
    if (!args || !bytes) return PDN_EINVAL;
    try {
        // validate everything except the workspace itself, then size it (the
        // size arithmetic relies on the validated bounds)
        const int rc = check_chunk(args, false);
        if (rc != PDN_OK) return rc;
        *bytes = pdn::chunk_fwd_workspace_bytes(*args);
        return PDN_OK;
    } catch (...) {
        return PDN_EINVAL;
    }
}

int pdn_chunk_fwd_check(const pdn_chunk_fwd_args* args) {
    try {
        return check_chunk(args);
    } catch (...) {
        return PDN_EINVAL;
    }
}

int pdn_chunk_fwd(const pdn_chunk_fwd_args* args, void* stream) {
    try {
        const int rc = check_chunk(args);
        if (rc != PDN_OK) return rc;
        const hipError_t e = pdn::launch_chunk_fwd(*args, static_cast<hipStream_t>(stream));
        if (e == hipErrorNotSupported) return PDN_EUNSUPPORTED;
        return e == hipSuccess ? PDN_OK : PDN_EHIP;
    } catch (...) {
        return PDN_EHIP;
    }
}

int pdn_chunk_fwd_noalloc(const pdn_chunk_fwd_args* args, void* stream) {
    try {
        int rc = check_chunk(args, false);
        if (rc != PDN_OK) return rc;
        pdn_chunk_fwd_args a = *args;
        const size_t need = pdn::chunk_fwd_workspace_bytes(a);
        if (need > PDN_NOALLOC_SCRATCH_BYTES) return PDN_ESCRATCH;
        a.workspace = nullptr;
        a.workspace_bytes = 0;
        if (need > 0) {
            void* p = scratch_on_current_device();
            if (!p) return PDN_EHIP;
            a.workspace = p;
            a.workspace_bytes = PDN_NOALLOC_SCRATCH_BYTES;
        }
        const hipError_t e = pdn::launch_chunk_fwd(a, static_cast<hipStream_t>(stream));
        if (e == hipErrorNotSupported) return PDN_EUNSUPPORTED;
        return e == hipSuccess ? PDN_OK : PDN_EHIP;
    } catch (...) {
        return PDN_EHIP;
    }
}

int pdn_chunk_bwd_workspace_size(const pdn_chunk_bwd_args* args, size_t* bytes) {
    if (!args || !bytes) return PDN_EINVAL;
    try {
        const int rc = check_bwd(args, false);
        if (rc != PDN_OK) return rc;
        *bytes = pdn::chunk_bwd_workspace_bytes(*args);
        return PDN_OK;
    } catch (...) {
        return PDN_EINVAL;
    }
}

int pdn_chunk_bwd_check(const pdn_chunk_bwd_args* args) {
    try {
        return check_bwd(args);
    } catch (...) {
        return PDN_EINVAL;
    }
}

int pdn_chunk_bwd(const pdn_chunk_bwd_args* args, void* stream) {
    try {
        const int rc = check_bwd(args);
        if (rc != PDN_OK) return rc;
        const hipError_t e = pdn::launch_chunk_bwd(*args, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? PDN_OK : PDN_EHIP;
    } catch (...) {
        return PDN_EHIP;
    }
}

int pdn_decode_check(const pdn_decode_args* args) {
    try {
        return check_decode(args);
    } catch (...) {
        return PDN_EINVAL;
    }
}

int pdn_decode_step(const pdn_decode_args* args, void* stream) {
    try {
        const int rc = check_decode(args);
        if (rc != PDN_OK) return rc;
        const hipError_t e = pdn::launch_decode(*args, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? PDN_OK : PDN_EHIP;
    } catch (...) {
        return PDN_EHIP;
    }
}

}  // extern "C"
