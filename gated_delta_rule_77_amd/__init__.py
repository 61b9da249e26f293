"""MI355X (gfx950) gated delta-rule library: Python binding of libpdn.so.

This layer only marshals arguments: it checks tensor placement, dtypes and
shapes, passes raw device pointers and the current HIP stream to the C ABI
(include/pdn.h), and raises on a non-zero return code.  Every step of the
computation runs in the HIP kernels of libpdn.so; there is no fallback, and
loading fails loudly when the library is missing.

PyTorch is used for device memory and streams only.

Entry points (same names as the C ABI):
    pdn_chunk_fwd(...)                 prefill over [B,H,T,d]
    pdn_chunk_fwd_noalloc(...)         the same with the library's static scratch
    pdn_chunk_fwd_workspace_size(...)  scratch bytes the prefill needs
    pdn_decode_step(...)               one token against a resident state
    pdn_chunk_bwd(...)                 gradients of the prefill
    pdn_chunk_bwd_workspace_size(...)  scratch bytes the backward needs
    pdn_abi_version(), pdn_strerror(code)
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpdn.so")

# The argument structs below mirror this version of include/pdn.h.
PDN_ABI_VERSION = 5

PDN_OK, PDN_EINVAL, PDN_EUNSUPPORTED, PDN_EWORKSPACE, PDN_EHIP, PDN_ESCRATCH = 0, -1, -2, -3, -4, -5
PDN_NOALLOC_SCRATCH_BYTES = 256 << 20   # static scratch of pdn_chunk_fwd_noalloc
PDN_F32, PDN_BF16 = 0, 1
PDN_ALPHA_NONE, PDN_ALPHA_SCALAR, PDN_ALPHA_VEC = 0, 1, 2
PDN_GATE_SCALAR, PDN_GATE_VEC, PDN_GAMMA_SAME_AS_BETA = 1, 2, 3
PDN_KEY_SYMMETRIC, PDN_KEY_ERASE_GATE, PDN_KEY_WRITE_GATE = 0, 1, 2
PDN_PRECOND_INVERSE, PDN_PRECOND_STABILISED = 0, 1

_P = ctypes.c_void_p
_I = ctypes.c_int32


class ChunkFwdArgs(ctypes.Structure):
    """Mirror of ``pdn_chunk_fwd_args``."""
    _fields_ = [("B", _I), ("H", _I), ("T", _I), ("dk", _I), ("dv", _I),
                ("qkv_dtype", _I), ("o_dtype", _I),
                ("q", _P), ("k", _P), ("v", _P),
                ("alpha_mode", _I), ("log_alpha", _P),
                ("beta_mode", _I), ("beta", _P),
                ("gamma_mode", _I), ("gamma", _P),
                ("key_mode", _I),
                ("precond_eps", ctypes.c_float), ("precond_mode", _I), ("precond_x", ctypes.c_float),
                ("precond_A0", _P), ("precond_AT", _P),
                ("S0", _P), ("ST", _P), ("o", _P),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class ChunkBwdArgs(ctypes.Structure):
    """Mirror of ``pdn_chunk_bwd_args``."""
    _fields_ = [("fwd", ChunkFwdArgs), ("dO", _P), ("dST", _P),
                ("dq", _P), ("dk", _P), ("dv", _P),
                ("dlog_alpha", _P), ("dbeta", _P), ("dgamma", _P),
                ("dS0", _P), ("dA0", _P),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class DecodeArgs(ctypes.Structure):
    """Mirror of ``pdn_decode_args``."""
    _fields_ = [("B", _I), ("H", _I), ("dk", _I), ("dv", _I),
                ("qkv_dtype", _I), ("o_dtype", _I),
                ("q", _P), ("k", _P), ("v", _P),
                ("alpha_mode", _I), ("log_alpha", _P),
                ("beta_mode", _I), ("beta", _P),
                ("gamma_mode", _I), ("gamma", _P),
                ("key_mode", _I),
                ("precond_eps", ctypes.c_float), ("precond_mode", _I), ("precond_x", ctypes.c_float),
                ("precond_A", _P),
                ("S", _P), ("o", _P)]


EXPORTED = ("pdn_abi_version", "pdn_strerror", "pdn_chunk_fwd_workspace_size",
            "pdn_chunk_fwd_check", "pdn_chunk_fwd", "pdn_chunk_fwd_noalloc", "pdn_decode_check",
            "pdn_decode_step", "pdn_chunk_bwd_workspace_size", "pdn_chunk_bwd_check",
            "pdn_chunk_bwd")

_lib = None
_lock = threading.Lock()


class PdnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (where, pdn_strerror(code), code))


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libpdn.so (built by ``gated_delta_rule_77_amd.build``); raise if absent."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError("libpdn.so not found at %s: build it with "
                               "`python -m gated_delta_rule_77_amd.build` (there is no "
                               "fallback implementation)" % p)
        lib = ctypes.CDLL(p)
        lib.pdn_abi_version.argtypes = []
        lib.pdn_abi_version.restype = ctypes.c_int
        lib.pdn_strerror.argtypes = [ctypes.c_int]
        lib.pdn_strerror.restype = ctypes.c_char_p
        lib.pdn_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(ChunkFwdArgs),
                                                     ctypes.POINTER(ctypes.c_size_t)]
        lib.pdn_chunk_fwd_workspace_size.restype = ctypes.c_int
        lib.pdn_chunk_fwd_check.argtypes = [ctypes.POINTER(ChunkFwdArgs)]
        lib.pdn_chunk_fwd_check.restype = ctypes.c_int
        lib.pdn_chunk_fwd.argtypes = [ctypes.POINTER(ChunkFwdArgs), _P]
        lib.pdn_chunk_fwd.restype = ctypes.c_int
        lib.pdn_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkFwdArgs), _P]
        lib.pdn_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.pdn_chunk_bwd_workspace_size.argtypes = [ctypes.POINTER(ChunkBwdArgs),
                                                     ctypes.POINTER(ctypes.c_size_t)]
        lib.pdn_chunk_bwd_workspace_size.restype = ctypes.c_int
        lib.pdn_chunk_bwd_check.argtypes = [ctypes.POINTER(ChunkBwdArgs)]
        lib.pdn_chunk_bwd_check.restype = ctypes.c_int
        lib.pdn_chunk_bwd.argtypes = [ctypes.POINTER(ChunkBwdArgs), _P]
        lib.pdn_chunk_bwd.restype = ctypes.c_int
        lib.pdn_decode_check.argtypes = [ctypes.POINTER(DecodeArgs)]
        lib.pdn_decode_check.restype = ctypes.c_int
        lib.pdn_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _P]
        lib.pdn_decode_step.restype = ctypes.c_int
        # a library built from another header version would read the
        # argument structs at other offsets (device pointers included)
        ver = int(lib.pdn_abi_version())
        if ver != PDN_ABI_VERSION:
            raise RuntimeError("%s has ABI version %d, this binding mirrors version %d: "
                               "rebuild it with `python -m gated_delta_rule_77_amd.build`"
                               % (p, ver, PDN_ABI_VERSION))
        if path is None:
            _lib = lib
        return lib


def pdn_abi_version() -> int:
    return int(load_library().pdn_abi_version())


def pdn_strerror(code: int) -> str:
    return load_library().pdn_strerror(int(code)).decode()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t):
    """Device pointer of a contiguous torch tensor (or None / raw int)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _qkv_dtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return PDN_BF16
    if t.dtype == torch.float32:
        return PDN_F32
    raise ValueError("q/k/v/o must be float32 or bfloat16, got %s" % t.dtype)


def _f32(t, name):
    import torch
    if t is None:
        return
    if t.dtype != torch.float32:
        raise ValueError("%s must be float32" % name)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _shape(t, name, *allowed):
    """Raise unless tensor t (None allowed only when None is listed) has one
    of the allowed shapes.  The C ABI receives bare pointers and cannot know
    a tensor's extent, so a wrongly shaped tensor would be read (or written)
    past its end: every tensor is checked here before a pointer is taken."""
    if t is None:
        if None in allowed:
            return
        raise ValueError("%s is required" % name)
    shapes = [a for a in allowed if a is not None]
    if tuple(t.shape) not in shapes:
        raise ValueError("%s must have shape %s, got %s" % (
            name, " or ".join("[%s]" % ",".join(str(x) for x in a) for a in shapes),
            list(t.shape)))


def _same_device(ref, named):
    """Every tensor must live on the device of `ref` (q)."""
    for name, t in named:
        if t is not None and not isinstance(t, int) and t.device != ref.device:
            raise ValueError("%s is on %s, q on %s: every tensor must share q's device"
                             % (name, t.device, ref.device))


def _alpha_mode(log_alpha, lead):
    if log_alpha is None:
        return PDN_ALPHA_NONE
    return PDN_ALPHA_SCALAR if log_alpha.dim() == lead else PDN_ALPHA_VEC


def _gate_mode(g, lead):
    return PDN_GATE_SCALAR if g.dim() == lead else PDN_GATE_VEC


def _precond_fields(a, precond_eps, precond_mode, precond_x):
    a.precond_eps = -1.0 if precond_eps is None else float(precond_eps)
    a.precond_mode = int(precond_mode)
    a.precond_x = float(precond_x)


def _chunk_args(q, k, v, o, log_alpha, beta, gamma, precond_eps, precond_A0,
                precond_AT, S0, ST, workspace, key_mode, precond_mode=PDN_PRECOND_INVERSE,
                precond_x=1.5):
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if tuple(k.shape) != (B, H, T, dk) or tuple(v.shape[:3]) != (B, H, T):
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    _shape(o, "o", (B, H, T, dv))
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share one dtype")
    _shape(log_alpha, "log_alpha", None, (B, H, T), (B, H, T, dk))
    _shape(beta, "beta", (B, H, T), (B, H, T, dk))
    _shape(gamma, "gamma", None, (B, H, T), (B, H, T, dv))
    _shape(precond_A0, "precond_A0", None, (B, H, dk))
    _shape(precond_AT, "precond_AT", None, (B, H, dk))
    _shape(S0, "S0", None, (B, H, dk, dv))
    _shape(ST, "ST", None, (B, H, dk, dv))
    _same_device(q, (("k", k), ("v", v), ("o", o), ("log_alpha", log_alpha), ("beta", beta),
                     ("gamma", gamma), ("precond_A0", precond_A0),
                     ("precond_AT", precond_AT), ("S0", S0), ("ST", ST),
                     ("workspace", workspace)))
    for name, t in (("log_alpha", log_alpha), ("beta", beta), ("gamma", gamma),
                    ("precond_A0", precond_A0), ("precond_AT", precond_AT),
                    ("S0", S0), ("ST", ST)):
        _f32(t, name)
    a = ChunkFwdArgs()
    a.B, a.H, a.T, a.dk, a.dv = B, H, T, dk, dv
    a.qkv_dtype, a.o_dtype = _qkv_dtype(q), _qkv_dtype(o)
    a.q, a.k, a.v, a.o = _ptr(q), _ptr(k), _ptr(v), _ptr(o)
    a.alpha_mode = _alpha_mode(log_alpha, 3)
    a.log_alpha = _ptr(log_alpha)
    a.beta_mode = _gate_mode(beta, 3)
    a.beta = _ptr(beta)
    a.gamma_mode = PDN_GAMMA_SAME_AS_BETA if gamma is None else _gate_mode(gamma, 3)
    a.gamma = _ptr(gamma)
    a.key_mode = int(key_mode)
    _precond_fields(a, precond_eps, precond_mode, precond_x)
    a.precond_A0, a.precond_AT = _ptr(precond_A0), _ptr(precond_AT)
    a.S0, a.ST = _ptr(S0), _ptr(ST)
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def pdn_chunk_fwd_workspace_size(q, k, v, o, log_alpha=None, beta=None, gamma=None,
                                 precond_eps=None, precond_A0=None, precond_AT=None,
                                 S0=None, ST=None, key_mode=PDN_KEY_SYMMETRIC,
                                 precond_mode=PDN_PRECOND_INVERSE, precond_x=1.5) -> int:
    a = _chunk_args(q, k, v, o, log_alpha, beta, gamma, precond_eps, precond_A0,
                    precond_AT, S0, ST, None, key_mode, precond_mode, precond_x)
    n = ctypes.c_size_t(0)
    rc = load_library().pdn_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if rc != PDN_OK:
        raise PdnError(rc, "pdn_chunk_fwd_workspace_size")
    return int(n.value)


def pdn_chunk_fwd(q, k, v, o, log_alpha=None, beta=None, gamma=None, precond_eps=None,
                  precond_A0=None, precond_AT=None, S0=None, ST=None, workspace=None,
                  stream=None, key_mode=PDN_KEY_SYMMETRIC, precond_mode=PDN_PRECOND_INVERSE,
                  precond_x=1.5) -> None:
    """Prefill.  Tensors are device tensors in the layouts of include/pdn.h.

    The gate modes follow from the tensors' ranks: log_alpha None / [B,H,T] /
    [B,H,T,dk]; beta [B,H,T] / [B,H,T,dk]; gamma None (same as beta) / [B,H,T]
    / [B,H,T,dv].  key_mode is one of PDN_KEY_*; precond_mode one of
    PDN_PRECOND_* (precond_x is the stabilised mode's bound).  o (float32 or
    bfloat16) receives the output; ST and
    precond_AT, when given, receive the final state and running k(.)k sum.
    workspace: a device tensor of at least pdn_chunk_fwd_workspace_size() bytes.
    When None and the call needs one, it is allocated here with torch's caching
    allocator, whose stream-ordered reuse makes that safe on torch's current
    stream; pass one explicitly when launching on another stream.
    """
    a = _chunk_args(q, k, v, o, log_alpha, beta, gamma, precond_eps, precond_A0,
                    precond_AT, S0, ST, workspace, key_mode, precond_mode, precond_x)
    lib = load_library()
    if workspace is None:
        n = ctypes.c_size_t(0)
        rc = lib.pdn_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
        if rc != PDN_OK:
            raise PdnError(rc, "pdn_chunk_fwd_workspace_size")
        if n.value:
            import torch
            workspace = torch.empty(int(n.value), dtype=torch.uint8, device=q.device)
            a.workspace = _ptr(workspace)
            a.workspace_bytes = int(n.value)
    rc = lib.pdn_chunk_fwd(ctypes.byref(a), _stream(stream))
    if rc != PDN_OK:
        raise PdnError(rc, "pdn_chunk_fwd")


def pdn_chunk_fwd_noalloc(q, k, v, o, log_alpha=None, beta=None, gamma=None, precond_eps=None,
                          precond_A0=None, precond_AT=None, S0=None, ST=None, stream=None,
                          key_mode=PDN_KEY_SYMMETRIC, precond_mode=PDN_PRECOND_INVERSE,
                          precond_x=1.5) -> None:
    """pdn_chunk_fwd without a workspace argument and without any allocation:
    the scratch comes from the library's static per-GPU array of
    PDN_NOALLOC_SCRATCH_BYTES (PdnError with PDN_ESCRATCH when the call needs
    more).  For callers that cannot allocate, e.g. under HIP graph capture.
    Calls on one GPU share that array: they must not overlap."""
    a = _chunk_args(q, k, v, o, log_alpha, beta, gamma, precond_eps, precond_A0,
                    precond_AT, S0, ST, None, key_mode, precond_mode, precond_x)
    rc = load_library().pdn_chunk_fwd_noalloc(ctypes.byref(a), _stream(stream))
    if rc != PDN_OK:
        raise PdnError(rc, "pdn_chunk_fwd_noalloc")


def _bwd_args(q, k, v, dO, dq, dk, dv, dlog_alpha, dbeta, dgamma, dS0, dA0, log_alpha, beta,
              gamma, precond_eps, precond_A0, S0, dST, workspace, key_mode, precond_mode,
              precond_x):
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dkk = q.shape
    dvv = v.shape[-1]
    if tuple(dq.shape) != (B, H, T, dkk) or tuple(dk.shape) != (B, H, T, dkk):
        raise ValueError("dq, dk must be [B,H,T,dk]")
    if tuple(dv.shape) != (B, H, T, dvv):
        raise ValueError("dv must be [B,H,T,dv]")
    _shape(dST, "dST", None, (B, H, dkk, dvv))
    _shape(dS0, "dS0", None, (B, H, dkk, dvv))
    _shape(dA0, "dA0", None, (B, H, dkk))
    _same_device(q, (("dO", dO), ("dST", dST), ("dq", dq), ("dk", dk), ("dv", dv),
                     ("dlog_alpha", dlog_alpha), ("dbeta", dbeta), ("dgamma", dgamma),
                     ("dS0", dS0), ("dA0", dA0), ("workspace", workspace)))
    for name, t, like in (("dlog_alpha", dlog_alpha, log_alpha), ("dbeta", dbeta, beta),
                          ("dgamma", dgamma, gamma)):
        if (t is None) != (like is None):
            raise ValueError("%s must be given exactly when its gate is" % name)
        if t is not None and tuple(t.shape) != tuple(like.shape):
            raise ValueError("%s must have the shape of its gate" % name)
    f = _chunk_args(q, k, v, dO, log_alpha, beta, gamma, precond_eps, precond_A0, None, S0,
                    None, None, key_mode, precond_mode, precond_x)
    f.o = None
    for name, t in (("dO", dO), ("dST", dST), ("dq", dq), ("dk", dk), ("dv", dv),
                    ("dlog_alpha", dlog_alpha), ("dbeta", dbeta), ("dgamma", dgamma),
                    ("dS0", dS0), ("dA0", dA0)):
        _f32(t, name)
    a = ChunkBwdArgs()
    a.fwd = f
    a.dO, a.dST = _ptr(dO), _ptr(dST)
    a.dq, a.dk, a.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    a.dlog_alpha, a.dbeta, a.dgamma = _ptr(dlog_alpha), _ptr(dbeta), _ptr(dgamma)
    a.dS0, a.dA0 = _ptr(dS0), _ptr(dA0)
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def pdn_chunk_bwd_workspace_size(q, k, v, dO, dq, dk, dv, dlog_alpha=None, dbeta=None,
                                 dgamma=None, dS0=None, dA0=None, log_alpha=None, beta=None,
                                 gamma=None, precond_eps=None, precond_A0=None, S0=None,
                                 dST=None, key_mode=PDN_KEY_SYMMETRIC,
                                 precond_mode=PDN_PRECOND_INVERSE, precond_x=1.5) -> int:
    a = _bwd_args(q, k, v, dO, dq, dk, dv, dlog_alpha, dbeta, dgamma, dS0, dA0, log_alpha,
                  beta, gamma, precond_eps, precond_A0, S0, dST, None, key_mode, precond_mode,
                  precond_x)
    n = ctypes.c_size_t(0)
    rc = load_library().pdn_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if rc != PDN_OK:
        raise PdnError(rc, "pdn_chunk_bwd_workspace_size")
    return int(n.value)


def pdn_chunk_bwd(q, k, v, dO, dq, dk, dv, dlog_alpha=None, dbeta=None, dgamma=None,
                  dS0=None, dA0=None, log_alpha=None, beta=None, gamma=None, precond_eps=None,
                  precond_A0=None, S0=None, dST=None, workspace=None, stream=None,
                  key_mode=PDN_KEY_SYMMETRIC, precond_mode=PDN_PRECOND_INVERSE,
                  precond_x=1.5) -> None:
    """Backward of the prefill: writes the gradients of
    sum <dO, o> + <dST, S_T> into the caller's fp32 tensors dq, dk [B,H,T,dk],
    dv [B,H,T,dv], dlog_alpha / dbeta / dgamma (shapes of their gates; given
    exactly when the gate is), dS0 [B,H,dk,dv] and dA0 [B,H,dk] (optional).
    The forward inputs are passed as to pdn_chunk_fwd.  workspace as for
    pdn_chunk_fwd (allocated here from torch's caching allocator when None).
    """
    a = _bwd_args(q, k, v, dO, dq, dk, dv, dlog_alpha, dbeta, dgamma, dS0, dA0, log_alpha,
                  beta, gamma, precond_eps, precond_A0, S0, dST, workspace, key_mode,
                  precond_mode, precond_x)
    lib = load_library()
    if workspace is None:
        n = ctypes.c_size_t(0)
        rc = lib.pdn_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
        if rc != PDN_OK:
            raise PdnError(rc, "pdn_chunk_bwd_workspace_size")
        if n.value:
            import torch
            workspace = torch.empty(int(n.value), dtype=torch.uint8, device=q.device)
            a.workspace = _ptr(workspace)
            a.workspace_bytes = int(n.value)
    rc = lib.pdn_chunk_bwd(ctypes.byref(a), _stream(stream))
    if rc != PDN_OK:
        raise PdnError(rc, "pdn_chunk_bwd")


def _decode_args(q, k, v, o, S, log_alpha, beta, gamma, precond_eps, precond_A, key_mode,
                 precond_mode=PDN_PRECOND_INVERSE, precond_x=1.5):
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k must be [B,H,dk] and v [B,H,dv]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    if tuple(k.shape) != (B, H, dk) or tuple(v.shape[:2]) != (B, H):
        raise ValueError("q, k must be [B,H,dk] and v [B,H,dv]")
    if tuple(o.shape) != (B, H, dv) or tuple(S.shape) != (B, H, dk, dv):
        raise ValueError("o must be [B,H,dv] and S [B,H,dk,dv]")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share one dtype")
    _shape(log_alpha, "log_alpha", None, (B, H), (B, H, dk))
    _shape(beta, "beta", (B, H), (B, H, dk))
    _shape(gamma, "gamma", None, (B, H), (B, H, dv))
    _shape(precond_A, "precond_A", None, (B, H, dk))
    _same_device(q, (("k", k), ("v", v), ("o", o), ("S", S), ("log_alpha", log_alpha),
                     ("beta", beta), ("gamma", gamma), ("precond_A", precond_A)))
    for name, t in (("log_alpha", log_alpha), ("beta", beta), ("gamma", gamma),
                    ("precond_A", precond_A), ("S", S)):
        _f32(t, name)
    a = DecodeArgs()
    a.B, a.H, a.dk, a.dv = B, H, dk, dv
    a.qkv_dtype, a.o_dtype = _qkv_dtype(q), _qkv_dtype(o)
    a.q, a.k, a.v, a.o, a.S = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(S)
    a.alpha_mode = _alpha_mode(log_alpha, 2)
    a.log_alpha = _ptr(log_alpha)
    a.beta_mode = _gate_mode(beta, 2)
    a.beta = _ptr(beta)
    a.gamma_mode = PDN_GAMMA_SAME_AS_BETA if gamma is None else _gate_mode(gamma, 2)
    a.gamma = _ptr(gamma)
    a.key_mode = int(key_mode)
    _precond_fields(a, precond_eps, precond_mode, precond_x)
    a.precond_A = _ptr(precond_A)
    return a


def pdn_decode_step(q, k, v, o, S, log_alpha=None, beta=None, gamma=None,
                    precond_eps=None, precond_A=None, stream=None,
                    key_mode=PDN_KEY_SYMMETRIC, precond_mode=PDN_PRECOND_INVERSE,
                    precond_x=1.5) -> None:
    """One decode token for all (b,h); S (and precond_A) updated in place."""
    a = _decode_args(q, k, v, o, S, log_alpha, beta, gamma, precond_eps, precond_A,
                     key_mode, precond_mode, precond_x)
    rc = load_library().pdn_decode_step(ctypes.byref(a), _stream(stream))
    if rc != PDN_OK:
        raise PdnError(rc, "pdn_decode_step")
