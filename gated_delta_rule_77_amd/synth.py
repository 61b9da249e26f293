"""Seeded synthetic inputs for the delta-rule recurrence.

This module only draws random numbers and shapes them into the workloads the
pages evaluate on (L2-normalised queries and keys, Gaussian values, sigmoid
gains, log-sigmoid-style decays, planted key/value pairs for retrieval).  It
holds none of the recurrence's arithmetic: the decay is handed over as its
natural log, the gains as given, and nothing here forms k*sqrt(beta), cumulative
sums, preconditioners or states.  Both the oracle tests and the GPU path take
their inputs from here, so this file must stay free of either side's code.

Every generator is deterministic in its seed (numpy PCG64).  Values that the
GPU receives in bf16 are rounded here (round-to-nearest-even) and returned as
float32 arrays that hold exactly those bf16 values, so the oracle and the GPU
see bit-identical inputs.

Workloads (pages: "Gated DeltaNet-2" technical summary; "FG^2-GDN" sections
2.1-2.3; "Preconditioned DeltaNet" section 2.2 (ja) / 2B (fr)):

* ``deltanet_fp32``   plain DeltaNet, fp32, B1 H1 T256 d64, alpha == 1.
* ``gdn``             Gated DeltaNet, bf16 q/k/v, scalar decay and gain.
* ``kda_fg2``         channel-wise decay, key-side vector gain, value gain =
                      mean of the key gain (FG^2 / KDA style).
* ``gdn2_precond``    decoupled erase/write vector gains, diagonal
                      preconditioner, planted key/value pairs (NIAH-shaped).
* ``decode``          resident fp32 state and per-step single-token inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# Gate-mode codes shared with the C ABI (include/pdn.h).  They are plain
# enumerations of how a gate tensor is shaped, not arithmetic.
ALPHA_NONE, ALPHA_SCALAR, ALPHA_VEC = 0, 1, 2
GATE_SCALAR, GATE_VEC, GAMMA_SAME_AS_BETA = 1, 2, 3
DT_F32, DT_BF16 = 0, 1


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even).

    Returns float32 values that are exactly representable in bf16.
    Inputs here are finite, so no NaN handling is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _neg_softplus(x: np.ndarray) -> np.ndarray:
    """log(exp(-softplus(x))) = -softplus(x), computed stably in float64."""
    x = x.astype(np.float64)
    sp = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    return (-sp).astype(np.float32)


@dataclass
class Workload:
    """One batch of inputs in the layout the C ABI takes.

    q, k: [B,H,T,dk]; v: [B,H,T,dv]; all float32 arrays (bf16-exact when
    ``qkv_dtype`` is bf16).  log_alpha: None, [B,H,T] or [B,H,T,dk].
    beta: [B,H,T] or [B,H,T,dk].  gamma: None (same as beta), [B,H,T] or
    [B,H,T,dv].  S0: None or [B,H,dk,dv].  A0: None or [B,H,dk].
    """

    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    qkv_dtype: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha_mode: int
    log_alpha: Optional[np.ndarray]
    beta_mode: int
    beta: np.ndarray
    gamma_mode: int
    gamma: Optional[np.ndarray]
    precond_eps: float = -1.0
    A0: Optional[np.ndarray] = None
    S0: Optional[np.ndarray] = None
    meta: Dict[str, object] = field(default_factory=dict)


def _qkv(rng, B, H, T, dk, dv, bf16):
    q = _l2_normalise(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    k = _l2_normalise(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    if bf16:
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def deltanet_fp32(B=1, H=1, T=256, d=64, seed=0) -> Workload:
    """Plain DeltaNet in fp32: alpha == 1, scalar beta, gamma = beta, S0 = 0."""
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, B, H, T, d, d, bf16=False)
    beta = _sigmoid(rng.standard_normal((B, H, T), dtype=np.float32))
    return Workload("deltanet_fp32", B, H, T, d, d, DT_F32, q, k, v,
                    ALPHA_NONE, None, GATE_SCALAR, beta, GAMMA_SAME_AS_BETA, None)


def gdn(B=4, H=16, T=4096, d=128, seed=0) -> Workload:
    """Gated DeltaNet: bf16 q/k/v; per-head scalar decay and gain, gamma = beta."""
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, B, H, T, d, d, bf16=True)
    log_alpha = _neg_softplus(rng.standard_normal((B, H, T), dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((B, H, T), dtype=np.float32))
    return Workload("gdn", B, H, T, d, d, DT_BF16, q, k, v,
                    ALPHA_SCALAR, log_alpha, GATE_SCALAR, beta, GAMMA_SAME_AS_BETA, None)


def kda_fg2(B=2, H=32, T=8192, d=128, seed=0) -> Workload:
    """Channel-wise decay, key-side vector gain, scalar value gain = mean(beta)."""
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, B, H, T, d, d, bf16=True)
    log_alpha = _neg_softplus(rng.standard_normal((B, H, T, d), dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((B, H, T, d), dtype=np.float32))
    gamma = beta.astype(np.float64).mean(axis=-1).astype(np.float32)
    return Workload("kda_fg2", B, H, T, d, d, DT_BF16, q, k, v,
                    ALPHA_VEC, log_alpha, GATE_VEC, beta, GATE_SCALAR, gamma)


def gdn2_precond(B=1, H=16, T=65536, d=128, seed=0, n_pairs=64,
                 eps=1e-6) -> Workload:
    """Decoupled erase/write vector gains with the diagonal preconditioner.

    n_pairs fresh key/value pairs are planted at distinct random positions in
    [0, T - n_pairs); the last n_pairs queries hold those keys in a random
    order, so a working memory returns the planted values there.
    """
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, B, H, T, d, d, bf16=False)
    log_alpha = _neg_softplus(rng.standard_normal((B, H, T, d), dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((B, H, T, d), dtype=np.float32))
    gamma = _sigmoid(rng.standard_normal((B, H, T, d), dtype=np.float32))
    n_pairs = min(n_pairs, max(T // 2, 0))
    positions = np.zeros((B, H, n_pairs), dtype=np.int64)
    perms = np.zeros((B, H, n_pairs), dtype=np.int64)
    if n_pairs > 0:
        for b in range(B):
            for h in range(H):
                pos = rng.choice(T - n_pairs, size=n_pairs, replace=False)
                kap = _l2_normalise(rng.standard_normal((n_pairs, d), dtype=np.float32))
                nu = rng.standard_normal((n_pairs, d), dtype=np.float32)
                perm = rng.permutation(n_pairs)
                k[b, h, pos] = kap
                v[b, h, pos] = nu
                q[b, h, T - n_pairs:] = kap[perm]
                positions[b, h] = pos
                perms[b, h] = perm
    q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return Workload("gdn2_precond", B, H, T, d, d, DT_BF16, q, k, v,
                    ALPHA_VEC, log_alpha, GATE_VEC, beta, GATE_VEC, gamma,
                    precond_eps=eps,
                    meta={"positions": positions, "perms": perms})


def decode(B=256, H=16, d=128, steps=1000, seed=0) -> Workload:
    """Recurrent decode: S0 ~ N(0, 0.02^2) fp32, then `steps` single tokens.

    Returned with T = steps (step-major draws reshaped to [B,H,T,...]); the
    decode entry point consumes one t at a time against the resident state.
    """
    rng = np.random.default_rng(seed)
    q = np.empty((B, H, steps, d), np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    la = np.empty_like(q)
    be = np.empty_like(q)
    for t in range(steps):
        q[:, :, t], k[:, :, t], v[:, :, t], la[:, :, t], be[:, :, t] = \
            _decode_step_draws(rng, B, H, d)
    q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    gamma = be.astype(np.float64).mean(axis=-1).astype(np.float32)
    S0 = (0.02 * rng.standard_normal((B, H, d, d), dtype=np.float32)).astype(np.float32)
    return Workload("decode", B, H, steps, d, d, DT_BF16, q, k, v,
                    ALPHA_VEC, la, GATE_VEC, be, GATE_SCALAR, gamma, S0=S0)


def _decode_step_draws(rng, B, H, d):
    q = _l2_normalise(rng.standard_normal((B, H, d), dtype=np.float32))
    k = _l2_normalise(rng.standard_normal((B, H, d), dtype=np.float32))
    v = rng.standard_normal((B, H, d), dtype=np.float32)
    la = _neg_softplus(rng.standard_normal((B, H, d), dtype=np.float32))
    be = _sigmoid(rng.standard_normal((B, H, d), dtype=np.float32))
    return q, k, v, la, be


def decode_stream(B=256, H=16, d=128, steps=1000, seed=0):
    """The ``decode`` workload without holding all steps in memory.

    Returns (S0, step_iter): S0 [B,H,d,d] as ``decode`` draws it, and an
    iterator over the steps yielding (q, k, v, log_alpha, beta, gamma), each
    [B,H,d] (gamma [B,H]), equal to ``decode(...)``'s slices at that step.
    ``decode`` draws S0 after all steps, so the stream runs the generator
    twice: once to reach S0, once to yield the steps.
    """
    rng = np.random.default_rng(seed)
    for _ in range(steps):
        _decode_step_draws(rng, B, H, d)
    S0 = (0.02 * rng.standard_normal((B, H, d, d), dtype=np.float32)).astype(np.float32)

    def steps_iter():
        r = np.random.default_rng(seed)
        for _ in range(steps):
            q, k, v, la, be = _decode_step_draws(r, B, H, d)
            gamma = be.astype(np.float64).mean(axis=-1).astype(np.float32)
            yield round_to_bf16(q), round_to_bf16(k), round_to_bf16(v), la, be, gamma
    return S0, steps_iter()


def headline(B=4, H=16, T=8192, d=128, seed=0) -> Workload:
    """The throughput workload: H=16, d=128, T=8K with Gated-DeltaNet gating."""
    w = gdn(B=B, H=H, T=T, d=d, seed=seed)
    w.name = "gdn_T8192"
    return w


def upstream_grads(w: Workload, seed: int = 1):
    """Seeded upstream gradients for the backward of a prefill workload:
    dO [B,H,T,dv] and dST [B,H,dk,dv], both N(0,1) float32 (the gradient of a
    loss that weighs every output and the final state alike)."""
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal((w.B, w.H, w.T, w.dv), dtype=np.float32)
    dST = rng.standard_normal((w.B, w.H, w.dk, w.dv), dtype=np.float32)
    return dO, dST


CONFIGS = {
    "deltanet_fp32": deltanet_fp32,
    "gdn": gdn,
    "kda_fg2": kda_fg2,
    "gdn2_precond": gdn2_precond,
    "decode": decode,
    "headline": headline,
}
