"""Alternative formulations of the delta-rule recurrence, used only to pin the
oracle (tests infrastructure; nothing in the product imports this file).

* ``unrolled_product`` -- explicit product of per-token transition matrices.
* ``chunked_wy``       -- chunkwise UT/WY form with a triangular solve.
* ``ridge_memory``, ``apply_to_key_exact``, ``apply_to_query_exact`` -- the
  exact-preconditioner references of "Preconditioned DeltaNet" (Theorem 3.1):
  the (ridge-regularised) least-squares memory and the two recurrences that
  reach it, DeltaNet with the inverse Gram matrix on the write key and linear
  attention with it on the query.

Both take the per-token gates from ``oracle._gates_per_token`` so that the
pins exercise the recurrence algebra; the gate definitions themselves are
pinned separately by closed forms in ``test_oracle.py``.
"""
import numpy as np

from oracle import ALPHA_NONE, ALPHA_SCALAR, ALPHA_VEC, GATE_SCALAR, GATE_VEC, GAMMA_SAME_AS_BETA
from oracle import KEY_SYMMETRIC
from oracle import _gates_per_token, _f64, keys_and_value


def unrolled_product(q, k, v, alpha_mode, log_alpha, beta_mode, beta, gamma_mode,
                     gamma, precond_eps=-1.0, A0=None, S0=None, key_mode=KEY_SYMMETRIC,
                     precond_mode=0, precond_x=1.5):
    """Explicit transition-matrix form for tiny inputs.

    With write key kw, read key kr and written value vw of each token (equal
    keys kt in the symmetric mode), M_t = (I - kw_t kr_t^T) Diag(alpha_t) and
    Phi_{t:s} = M_t ... M_s,
        S_t = Phi_{t:1} S_0 + sum_{s<=t} Phi_{t:s+1} kw_s vw_s^T,
    which is the closed form of the delta rule written as a diagonal-plus-
    low-rank linear recurrence (FG^2-GDN, 2.1 and 2.3).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    ST = np.zeros((B, H, dk, dv))
    I = np.eye(dk)
    for b in range(B):
        for h in range(H):
            sel = lambda x: None if x is None else _f64(x)[b, h]
            alpha, be, ga, _ = _gates_per_token(alpha_mode, sel(log_alpha), beta_mode,
                                                sel(beta), gamma_mode, sel(gamma),
                                                precond_eps, sel(A0), k[b, h], dk, dv,
                                                precond_mode, precond_x)
            kv = [keys_and_value(key_mode, be[t], ga[t], k[b, h, t], v[b, h, t],
                                 gamma_mode == GAMMA_SAME_AS_BETA) for t in range(T)]
            kts = [x[0] for x in kv]
            krs = [x[1] for x in kv]
            vts = [x[2] for x in kv]
            Ms = [(I - np.outer(kts[t], krs[t])) @ np.diag(alpha[t]) for t in range(T)]
            S0bh = np.zeros((dk, dv)) if S0 is None else _f64(S0)[b, h]
            for t in range(T):
                # Phi_{t:1}
                Phi = I.copy()
                for s in range(t + 1):
                    Phi = Ms[s] @ Phi
                St = Phi @ S0bh
                for s in range(t + 1):
                    P = I.copy()
                    for r in range(s + 1, t + 1):
                        P = Ms[r] @ P
                    St = St + P @ np.outer(kts[s], vts[s])
                o[b, h, t] = St.T @ q[b, h, t]
                if t == T - 1:
                    ST[b, h] = St
            if T == 0:
                ST[b, h] = S0bh
    return o, ST


def chunked_wy(q, k, v, alpha_mode, log_alpha, beta_mode, beta, gamma_mode,
               gamma, precond_eps=-1.0, A0=None, S0=None, C=16, key_mode=KEY_SYMMETRIC,
               precond_mode=0, precond_x=1.5):
    """Chunkwise-parallel form with a per-chunk unit-lower-triangular solve.

    Within a chunk (positions r = 1..C, cumulative log-decay G_r per key
    channel, Gamma_r = exp(G_r), write keys Kw, read keys Kr, written values
    Vw; Kw = Kr = Kt in the symmetric mode):
        T_rs = sum_i kr_ri kw_si exp(G_ri - G_si)            (s < r)
        P_rs = sum_i q_ri  kw_si exp(G_ri - G_si)            (s <= r)
        (I + T) U = Vw - (Kr (.) Gamma) S_0                    (forward solve)
        O = (Q (.) Gamma) S_0 + P U
        S_C = Diag(Gamma_C) S_0 + (Kw (.) exp(G_C - G))^T U
    This is the UT/WY chunk algorithm the pages describe (Gated DeltaNet-2,
    "chunk parallel training": the decay absorbed into the erase/write
    matrices and a lower-triangular (I+T)^-1 solve).  fp64, for pins only.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            sel = lambda x: None if x is None else _f64(x)[b, h]
            alpha, be, ga, _ = _gates_per_token(alpha_mode, sel(log_alpha), beta_mode,
                                                sel(beta), gamma_mode, sel(gamma),
                                                precond_eps, sel(A0), k[b, h], dk, dv,
                                                precond_mode, precond_x)
            logal = np.log(alpha)
            S = np.zeros((dk, dv)) if S0 is None else _f64(S0)[b, h].copy()
            for c0 in range(0, T, C):
                c1 = min(c0 + C, T)
                kv = [keys_and_value(key_mode, be[t], ga[t], k[b, h, t], v[b, h, t],
                                     gamma_mode == GAMMA_SAME_AS_BETA) for t in range(c0, c1)]
                Kt = np.array([x[0] for x in kv])
                Kr = np.array([x[1] for x in kv])
                Vt = np.array([x[2] for x in kv])
                Q = q[b, h, c0:c1]
                G = np.cumsum(logal[c0:c1], axis=0)
                n = c1 - c0
                Tm = np.zeros((n, n))
                Pm = np.zeros((n, n))
                for r in range(n):
                    for s in range(r + 1):
                        dec = np.exp(G[r] - G[s])
                        if s < r:
                            Tm[r, s] = np.sum(Kr[r] * Kt[s] * dec)
                        Pm[r, s] = np.sum(Q[r] * Kt[s] * dec)
                rhs = Vt - (Kr * np.exp(G)) @ S
                U = np.linalg.solve(np.eye(n) + Tm, rhs)
                o[b, h, c0:c1] = (Q * np.exp(G)) @ S + Pm @ U
                S = np.exp(G[-1])[:, None] * S + (Kt * np.exp(G[-1] - G)).T @ U
            ST[b, h] = S
    return o, ST


# ---------------------------------------------------------------------------
# exact preconditioner ("Preconditioned DeltaNet", Theorem 3.1)
# ---------------------------------------------------------------------------

def ridge_memory(k, v, lam):
    """Per prefix t, the memory S_t = argmin_S lam ||S||^2 + sum_{i<=t} ||S^T k_i - v_i||^2
    = (lam I + K_t^T K_t)^-1 K_t^T V_t, by a dense solve.  k [T, dk], v [T, dv] -> [T, dk, dv]."""
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    T, dk = k.shape
    out = np.zeros((T, dk, v.shape[1]))
    for t in range(T):
        K, V = k[:t + 1], v[:t + 1]
        out[t] = np.linalg.solve(lam * np.eye(dk) + K.T @ K, K.T @ V)
    return out


def apply_to_key_exact(q, k, v, lam):
    """DeltaNet with the exact preconditioner on the write key: read key k_t,
    write key G_t^-1 k_t with G_t = lam I + sum_{i<=t} k_i k_i^T, unit gain, no
    decay, S_0 = 0.  Returns (o [T, dv], S_T)."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    T, dk = k.shape
    G = lam * np.eye(dk)
    S = np.zeros((dk, v.shape[1]))
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        G += np.outer(k[t], k[t])
        kw = np.linalg.solve(G, k[t])
        S = S + np.outer(kw, v[t] - S.T @ k[t])
        o[t] = S.T @ q[t]
    return o, S


def apply_to_query_exact(q, k, v, lam):
    """Linear attention with the exact preconditioner on the query:
    o_t = sum_{i<=t} ((G_t^-1 q_t) . k_i) v_i, G_t as in apply_to_key_exact."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    T, dk = k.shape
    G = lam * np.eye(dk)
    M = np.zeros((dk, v.shape[1]))  # sum k_i v_i^T
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        G += np.outer(k[t], k[t])
        M += np.outer(k[t], v[t])
        o[t] = M.T @ np.linalg.solve(G, q[t])
    return o


def axis_key_case(rng, T, dk, dv, n_axes):
    """Keys along coordinate axes (random axis among the first n_axes, random
    bf16-exact magnitude), so every Gram matrix sum k k^T is diagonal."""
    axis = rng.integers(0, n_axes, T)
    mag = rng.choice(np.array([0.25, 0.5, 0.75, 1.0, 1.5, 2.0]), T) * rng.choice([-1.0, 1.0], T)
    k = np.zeros((T, dk))
    k[np.arange(T), axis] = mag
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    return q, k, v
