"""ORACLE -- test infrastructure, not part of the product.

A plain fp64 CPU reference of the gated delta-rule recurrence, written from
the pages before any GPU code.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it; the GPU
library never does, and this package imports nothing from it.

* ``delta_rule``        -- the token-by-token recurrence (C, fp64, OpenMP over
                           (batch, head)), built from ``recurrence.c``.
* ``delta_rule_py``     -- the same recurrence as a numpy loop for tiny cases.
* ``delta_rule_bwd``    -- its backward pass (reverse mode through the token
                           recurrence, fp64, C): gradients of
                           sum <dO, o> + <dST, S_T> with respect to q, k, v,
                           the decay, the gains, S0 and A0.

Every function is pinned by tests in ``tests/test_oracle.py`` against closed
forms, invariants and two other formulations of the same recurrence kept in
``tests/formulations.py``; the backward by ``tests/test_oracle_bwd.py``
(finite differences of the forward in every mode, Euler identities, a closed
form, autodiff of the transition-product form).  Parity unpinned: the stabilised preconditioner
(``precond_mode=PRECOND_STABILISED``, "Preconditioned DeltaNet" Eq. 9).  The
pages give its steps (log of the running second moment, centring, the squash
r / (1 + |r|), an exponent mapping into [1/x, x]) but not the centring constant,
the base or the sign; the form here (centring on the channel mean of
ln(A + eps), B = x^-s) is a reading, pinned by its own closed forms only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "recurrence.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ALPHA_NONE, ALPHA_SCALAR, ALPHA_VEC = 0, 1, 2
GATE_SCALAR, GATE_VEC, GAMMA_SAME_AS_BETA = 1, 2, 3
KEY_SYMMETRIC, KEY_ERASE_GATE, KEY_WRITE_GATE = 0, 1, 2
PRECOND_INVERSE, PRECOND_STABILISED = 0, 1


def build(force: bool = False) -> str:
    """Compile recurrence.c with gcc (plain -O2, OpenMP, no fast-math): the
    library the tests use, portable to any x86-64 host."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


BASELINE_FLAGS = ["-O3", "-march=native", "-ffp-contract=off", "-fopenmp"]


def load_native(outdir: str):
    """The same source built with BASELINE_FLAGS into `outdir` (for timing the
    oracle as a CPU baseline on the machine it runs on; the arithmetic is the
    same: no fast-math, no contraction into fused multiply-adds).  Returns a
    library handle for the `lib=` argument of delta_rule."""
    so = os.path.join(outdir, "liboracle_native.so")
    subprocess.check_call(["gcc", *BASELINE_FLAGS, "-fPIC", "-shared", "-std=c99", _SRC,
                           "-o", so, "-lm"])
    return _configure(ctypes.CDLL(so))


def _configure(lib):
    f = lib.oracle_delta_rule
    P = ctypes.c_void_p
    I = ctypes.c_int
    f.argtypes = [I, I, I, I, I, P, P, P, I, P, I, P, I, P,
                  ctypes.c_double, P, P, P, P, P, I, I, ctypes.c_double]
    f.restype = I
    g = lib.oracle_delta_rule_bwd
    g.argtypes = [I, I, I, I, I, P, P, P, I, P, I, P, I, P, ctypes.c_double, P, P,
                  I, I, ctypes.c_double, P, P, P, P, P, P, P, P, P, P]
    g.restype = I
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def num_threads(lib=None) -> int:
    """OpenMP threads the oracle runs on (its parallelism is over (b, h))."""
    return int((lib or _load()).oracle_num_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def delta_rule(q, k, v, alpha_mode, log_alpha, beta_mode, beta, gamma_mode,
               gamma, precond_eps: float = -1.0, A0=None, S0=None,
               want_state: bool = True, key_mode: int = KEY_SYMMETRIC,
               precond_mode: int = PRECOND_INVERSE, precond_x: float = 1.5, lib=None):
    """Run the fp64 recurrence.  Returns (o, S_T, A_T) as float64 arrays.

    Shapes follow the C ABI: q, k [B,H,T,dk]; v [B,H,T,dv]; gates and
    ``key_mode`` and ``precond_mode`` / ``precond_x`` (the bound x of the
    stabilised coefficient) as in ``recurrence.c``.  A_T is None unless the
    preconditioner is on.  ``lib``: a handle from load_native (default: the
    library build() makes).
    """
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    la, be, ga = _f64(log_alpha), _f64(beta), _f64(gamma)
    A0, S0 = _f64(A0), _f64(S0)
    o = np.zeros((B, H, T, dv), np.float64)
    ST = np.zeros((B, H, dk, dv), np.float64) if want_state else None
    AT = np.zeros((B, H, dk), np.float64) if precond_eps >= 0 else None
    rc = lib.oracle_delta_rule(B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                               int(alpha_mode), _ptr(la), int(beta_mode), _ptr(be),
                               int(gamma_mode), _ptr(ga), float(precond_eps),
                               _ptr(A0), _ptr(AT), _ptr(S0), _ptr(ST), _ptr(o),
                               int(key_mode), int(precond_mode), float(precond_x))
    if rc != 0:
        raise ValueError("oracle_delta_rule failed with code %d" % rc)
    return o, ST, AT


def delta_rule_bwd(q, k, v, alpha_mode, log_alpha, beta_mode, beta, gamma_mode,
                   gamma, dO, dST=None, precond_eps: float = -1.0, A0=None, S0=None,
                   key_mode: int = KEY_SYMMETRIC, precond_mode: int = PRECOND_INVERSE,
                   precond_x: float = 1.5):
    """Gradients of L = sum <dO, o> + <dST, S_T> for the recurrence of
    ``delta_rule`` (same arguments; dST None means zero).

    Returns a dict of float64 arrays: dq, dk [B,H,T,dk]; dv [B,H,T,dv];
    dlog_alpha (shape of log_alpha, None without decay); dbeta (shape of
    beta); dgamma (shape of gamma, None when gamma is "same as beta", whose
    gradient is in dbeta); dS0 [B,H,dk,dv]; dA0 [B,H,dk] (None without the
    preconditioner).
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    la, be, ga = _f64(log_alpha), _f64(beta), _f64(gamma)
    A0, S0, dO, dST = _f64(A0), _f64(S0), _f64(dO), _f64(dST)
    out = {
        "dq": np.zeros((B, H, T, dk)), "dk": np.zeros((B, H, T, dk)),
        "dv": np.zeros((B, H, T, dv)),
        "dlog_alpha": None if alpha_mode == ALPHA_NONE else np.zeros(la.shape),
        "dbeta": np.zeros(be.shape),
        "dgamma": None if gamma_mode == GAMMA_SAME_AS_BETA else np.zeros(ga.shape),
        "dS0": np.zeros((B, H, dk, dv)),
        "dA0": np.zeros((B, H, dk)) if precond_eps >= 0 else None,
    }
    rc = lib.oracle_delta_rule_bwd(B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                   int(alpha_mode), _ptr(la), int(beta_mode), _ptr(be),
                                   int(gamma_mode), _ptr(ga), float(precond_eps),
                                   _ptr(A0), _ptr(S0), int(key_mode), int(precond_mode),
                                   float(precond_x), _ptr(dO), _ptr(dST),
                                   _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                   _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]),
                                   _ptr(out["dgamma"]), _ptr(out["dS0"]), _ptr(out["dA0"]))
    if rc != 0:
        raise ValueError("oracle_delta_rule_bwd failed with code %d" % rc)
    return out


def run_workload(w, S0="from_workload", want_state=True):
    """Convenience: run the oracle on a ``synth.Workload``-like object."""
    s0 = w.S0 if isinstance(S0, str) else S0
    return delta_rule(w.q, w.k, w.v, w.alpha_mode, w.log_alpha, w.beta_mode,
                      w.beta, w.gamma_mode, w.gamma, w.precond_eps, w.A0, s0,
                      want_state=want_state, key_mode=getattr(w, "key_mode", KEY_SYMMETRIC))


def keys_and_value(key_mode, b, g, k, v, gamma_same):
    """Write key, read key and written value of one token for a key mode
    (b: erase gain with the preconditioner folded in, g: value gain)."""
    if key_mode == KEY_SYMMETRIC:
        kw = np.sqrt(b) * k
        return kw, kw, np.sqrt(g) * v
    if key_mode == KEY_ERASE_GATE:
        return k, b * k, g * v
    if key_mode == KEY_WRITE_GATE:
        return b * k, k, (v if gamma_same else g * v)
    raise ValueError("unknown key mode %r" % (key_mode,))


def precond_coeff(A, eps, precond_mode=PRECOND_INVERSE, precond_x=1.5):
    """Preconditioner coefficient per key channel from the running second
    moment A [..., dk]: 1 / (A + eps), or the stabilised reading
    x^-(r / (1 + |r|)) with r = ln(A + eps) - mean over channels."""
    if precond_mode == PRECOND_INVERSE:
        return 1.0 / (A + eps)
    lg = np.log(A + eps)
    r = lg - lg.mean(axis=-1, keepdims=True)
    return np.exp(-(r / (1.0 + np.abs(r))) * np.log(precond_x))


def _gates_per_token(alpha_mode, log_alpha, beta_mode, beta, gamma_mode, gamma,
                     precond_eps, A0, k, dk, dv, precond_mode=PRECOND_INVERSE, precond_x=1.5):
    """Per-token decay, erase gain and write gain for one (b, h): [T, dk/dv]."""
    T = k.shape[0]
    if alpha_mode == ALPHA_NONE:
        alpha = np.ones((T, dk))
    elif alpha_mode == ALPHA_SCALAR:
        alpha = np.repeat(np.exp(log_alpha)[:, None], dk, axis=1)
    else:
        alpha = np.exp(log_alpha)
    b = np.repeat(beta[:, None], dk, axis=1) if beta_mode == GATE_SCALAR else beta.copy()
    if gamma_mode == GAMMA_SAME_AS_BETA:
        g = np.repeat(beta[:, None], dv, axis=1) if beta_mode == GATE_SCALAR else beta.copy()
    elif gamma_mode == GATE_SCALAR:
        g = np.repeat(gamma[:, None], dv, axis=1)
    else:
        g = gamma.copy()
    A_T = None
    if precond_eps >= 0:
        # A_t is the inclusive running sum of k (.) k, plus A0 when given.
        acc = np.cumsum(k * k, axis=0) + (0.0 if A0 is None else A0[None, :])
        if precond_mode == PRECOND_INVERSE:
            b = b / (acc + precond_eps)
        else:
            b = b * precond_coeff(acc, precond_eps, precond_mode, precond_x)
        A_T = acc[-1] if T > 0 else (np.zeros(dk) if A0 is None else A0.copy())
    return alpha, b, g, A_T


def delta_rule_py(q, k, v, alpha_mode, log_alpha, beta_mode, beta, gamma_mode,
                  gamma, precond_eps=-1.0, A0=None, S0=None, key_mode=KEY_SYMMETRIC,
                  precond_mode=PRECOND_INVERSE, precond_x=1.5):
    """Numpy token loop for tiny inputs (same definition as the C oracle)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    ST = np.zeros((B, H, dk, dv))
    AT = np.zeros((B, H, dk)) if precond_eps >= 0 else None
    for b in range(B):
        for h in range(H):
            sel = lambda x: None if x is None else _f64(x)[b, h]
            alpha, be, ga, aT = _gates_per_token(alpha_mode, sel(log_alpha), beta_mode,
                                                 sel(beta), gamma_mode, sel(gamma),
                                                 precond_eps, sel(A0), k[b, h], dk, dv,
                                                 precond_mode, precond_x)
            S = np.zeros((dk, dv)) if S0 is None else _f64(S0)[b, h].copy()
            for t in range(T):
                kw, kr, vw = keys_and_value(key_mode, be[t], ga[t], k[b, h, t], v[b, h, t],
                                            gamma_mode == GAMMA_SAME_AS_BETA)
                Ad = alpha[t][:, None] * S
                S = Ad + np.outer(kw, vw - Ad.T @ kr)
                o[b, h, t] = S.T @ q[b, h, t]
            ST[b, h] = S
            if AT is not None:
                AT[b, h] = aT
    return o, ST, AT


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor (0 if both are zero)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm((x - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
