"""Pins for the oracle's backward pass (CPU only).

The gradients of L = sum <dO, o> + <dST, S_T> are pinned against things that
do not share the backward's arithmetic:

* central finite differences of the (separately pinned) forward oracle, in
  every decay / gain / key / preconditioner mode, on tiny inputs, and on
  sampled entries of a sequence that crosses the backward's recomputation
  checkpoints;
* Euler's identity for the parts of L that are linear: L is linear in
  (v, S0) jointly and <dO, o> is linear in q, so sum v dv + sum S0 dS0 = L
  and sum q dq = <dO, o>, at any size;
* a closed form: with zero gains in the erase-gate mode nothing is written,
  S_t = Diag(Gamma_t) S0, and dq, dS0, d log_alpha follow by hand;
* reverse-mode automatic differentiation (torch, fp64) of the explicit
  transition-matrix product form of the recurrence.

Each is chosen so that a dropped term, a wrong sign, a transposed operand or
an off-by-one token in the backward fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import (ALPHA_NONE, ALPHA_SCALAR, ALPHA_VEC, GATE_SCALAR, GATE_VEC, GAMMA_SAME_AS_BETA,
                    KEY_ERASE_GATE, KEY_SYMMETRIC, KEY_WRITE_GATE, PRECOND_INVERSE,
                    PRECOND_STABILISED)


def _case(rng, T, dk, dv, amode, bmode, gmode, precond, B=1, H=1):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    k *= 0.8 / np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    la = None
    if amode == ALPHA_SCALAR:
        la = -np.log1p(np.exp(rng.standard_normal((B, H, T))))
    elif amode == ALPHA_VEC:
        la = -np.log1p(np.exp(rng.standard_normal((B, H, T, dk))))
    be = rng.uniform(0.2, 0.95, (B, H, T) if bmode == GATE_SCALAR else (B, H, T, dk))
    ga = None
    if gmode == GATE_SCALAR:
        ga = rng.uniform(0.2, 0.95, (B, H, T))
    elif gmode == GATE_VEC:
        ga = rng.uniform(0.2, 0.95, (B, H, T, dv))
    S0 = 0.5 * rng.standard_normal((B, H, dk, dv))
    A0 = rng.uniform(0.5, 2.0, (B, H, dk)) if precond is not None else None
    dO = rng.standard_normal((B, H, T, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    return dict(q=q, k=k, v=v, alpha_mode=amode, log_alpha=la, beta_mode=bmode, beta=be,
                gamma_mode=gmode, gamma=ga, S0=S0, A0=A0, dO=dO, dST=dST,
                precond_eps=(1e-3 if precond is not None else -1.0),
                precond_mode=(precond if precond is not None else PRECOND_INVERSE))


def _loss(c, key_mode, **over):
    a = dict(c)
    a.update(over)
    o, ST, _ = oracle.delta_rule(a["q"], a["k"], a["v"], a["alpha_mode"], a["log_alpha"],
                                 a["beta_mode"], a["beta"], a["gamma_mode"], a["gamma"],
                                 a["precond_eps"], a["A0"], a["S0"], key_mode=key_mode,
                                 precond_mode=a["precond_mode"])
    return float((o * a["dO"]).sum() + (ST * a["dST"]).sum())


def _grads(c, key_mode):
    return oracle.delta_rule_bwd(c["q"], c["k"], c["v"], c["alpha_mode"], c["log_alpha"],
                                 c["beta_mode"], c["beta"], c["gamma_mode"], c["gamma"],
                                 c["dO"], c["dST"], c["precond_eps"], c["A0"], c["S0"],
                                 key_mode=key_mode, precond_mode=c["precond_mode"])


# input name -> gradient name
PAIRS = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_alpha", "dlog_alpha"),
         ("beta", "dbeta"), ("gamma", "dgamma"), ("S0", "dS0"), ("A0", "dA0")]


def _fd_check(c, key_mode, sample=None, rng=None, h=1e-6):
    g = _grads(c, key_mode)
    worst = 0.0
    for name, gname in PAIRS:
        x = c[name]
        if x is None:
            assert g[gname] is None or gname == "dA0"
            continue
        idxs = list(np.ndindex(x.shape))
        if sample is not None and len(idxs) > sample:
            idxs = [idxs[i] for i in rng.choice(len(idxs), sample, replace=False)]
        for idx in idxs:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd = (_loss(c, key_mode, **{name: xp}) - _loss(c, key_mode, **{name: xm})) / (2 * h)
            err = abs(fd - g[gname][idx])
            worst = max(worst, err / (1.0 + abs(fd)))
            assert err <= 1e-6 * (1.0 + abs(fd)), (name, idx, fd, g[gname][idx])
    return worst


GATE_MODES = [(a, b, g) for a in (ALPHA_NONE, ALPHA_SCALAR, ALPHA_VEC)
              for b in (GATE_SCALAR, GATE_VEC)
              for g in (GAMMA_SAME_AS_BETA, GATE_SCALAR, GATE_VEC)]


@pytest.mark.parametrize("key_mode", [KEY_SYMMETRIC, KEY_ERASE_GATE, KEY_WRITE_GATE])
@pytest.mark.parametrize("precond", [None, PRECOND_INVERSE, PRECOND_STABILISED])
@pytest.mark.parametrize("amode,bmode,gmode", GATE_MODES)
def test_bwd_matches_finite_differences(amode, bmode, gmode, precond, key_mode):
    """Every gradient, every entry, central differences of the forward oracle."""
    rng = np.random.default_rng(hash((amode, bmode, gmode, precond, key_mode)) % 2**32)
    dv = 4 if gmode == GAMMA_SAME_AS_BETA and bmode == GATE_VEC else 3
    c = _case(rng, T=6, dk=4, dv=dv, amode=amode, bmode=bmode, gmode=gmode, precond=precond)
    _fd_check(c, key_mode)


@pytest.mark.parametrize("key_mode,precond", [(KEY_SYMMETRIC, None), (KEY_SYMMETRIC, PRECOND_INVERSE),
                                              (KEY_ERASE_GATE, PRECOND_STABILISED),
                                              (KEY_WRITE_GATE, None)])
def test_bwd_across_checkpoints(key_mode, precond):
    """T = 150 crosses the backward's 64-token recomputation checkpoints: sampled
    central differences of every input, B = H = 2."""
    rng = np.random.default_rng(7 + key_mode)
    c = _case(rng, T=150, dk=4, dv=3, amode=ALPHA_VEC, bmode=GATE_VEC, gmode=GATE_SCALAR,
              precond=precond, B=2, H=1)
    _fd_check(c, key_mode, sample=25, rng=rng)


@pytest.mark.parametrize("key_mode", [KEY_SYMMETRIC, KEY_ERASE_GATE, KEY_WRITE_GATE])
@pytest.mark.parametrize("amode,bmode,gmode,precond", [
    (ALPHA_SCALAR, GATE_SCALAR, GAMMA_SAME_AS_BETA, None),
    (ALPHA_VEC, GATE_VEC, GATE_VEC, PRECOND_INVERSE),
    (ALPHA_VEC, GATE_VEC, GATE_SCALAR, PRECOND_STABILISED)])
def test_bwd_euler_identities(amode, bmode, gmode, precond, key_mode):
    """L is linear in (v, S0) jointly and <dO, o> is linear in q (the gates do not
    depend on v, S0 or q): sum v dv + sum S0 dS0 = L and sum q dq = <dO, o>."""
    rng = np.random.default_rng(11)
    c = _case(rng, T=300, dk=16, dv=16, amode=amode, bmode=bmode, gmode=gmode, precond=precond,
              B=2, H=2)
    g = _grads(c, key_mode)
    L = _loss(c, key_mode)
    lin = float((c["v"] * g["dv"]).sum() + (c["S0"] * g["dS0"]).sum())
    assert abs(lin - L) <= 1e-10 * (1 + abs(L))
    Lo = _loss(c, key_mode, dST=np.zeros_like(c["dST"]))
    assert abs(float((c["q"] * g["dq"]).sum()) - Lo) <= 1e-10 * (1 + abs(Lo))


def test_bwd_closed_form_no_write():
    """Erase-gate keys with zero gains write nothing: S_t = Diag(Gamma_t) S0 with
    Gamma_t the running product of alpha.  Then dq_t = Diag(Gamma_t) S0 dO_t,
    dS0 = sum_t Diag(Gamma_t) q_t dO_t^T + Diag(Gamma_T) dST, and
    d log_alpha_s = sum_{t >= s} (q_t (.) Gamma_t (.) S0 dO_t) + Gamma_T (.) rowsum(S0 (.) dST);
    dk, dv are zero."""
    rng = np.random.default_rng(3)
    T, dk, dv = 40, 6, 5
    c = _case(rng, T=T, dk=dk, dv=dv, amode=ALPHA_VEC, bmode=GATE_VEC, gmode=GAMMA_SAME_AS_BETA,
              precond=None)
    # gamma "same as beta" needs dk == dv for a vector beta: a scalar zero beta
    c["beta_mode"], c["beta"] = GATE_SCALAR, np.zeros((1, 1, T))
    g = _grads(c, KEY_ERASE_GATE)
    Gam = np.exp(np.cumsum(c["log_alpha"][0, 0], axis=0))  # [T, dk]
    S0, q, dO, dST = c["S0"][0, 0], c["q"][0, 0], c["dO"][0, 0], c["dST"][0, 0]
    dq = (Gam[:, :, None] * S0[None]) @ dO[:, :, None]
    np.testing.assert_allclose(g["dq"][0, 0], dq[:, :, 0], rtol=1e-12, atol=1e-12)
    dS0 = sum(np.outer(Gam[t] * q[t], dO[t]) for t in range(T)) + Gam[-1][:, None] * dST
    np.testing.assert_allclose(g["dS0"][0, 0], dS0, rtol=1e-12, atol=1e-12)
    per_t = q * Gam * (S0 @ dO.T).T  # [T, dk]: q_t,i Gamma_t,i (S0 dO_t)_i
    tail = Gam[-1] * (S0 * dST).sum(axis=1)
    dla = np.cumsum(per_t[::-1], axis=0)[::-1] + tail[None]
    np.testing.assert_allclose(g["dlog_alpha"][0, 0], dla, rtol=1e-11, atol=1e-12)
    assert np.abs(g["dk"]).max() == 0.0 and np.abs(g["dv"]).max() == 0.0


def _torch_product_form(q, k, v, la, be, ga, S0, key_mode):
    """o_t and S_T from the explicit transition product
    S_t = (I - kw kr^T) Diag(alpha_t) S_{t-1} + kw vw^T (vector gates), in torch."""
    T, dk = q.shape
    S = S0
    outs = []
    for t in range(T):
        a = torch.exp(la[t])
        if key_mode == KEY_SYMMETRIC:
            kw = torch.sqrt(be[t]) * k[t]
            kr = kw
            vw = torch.sqrt(ga[t]) * v[t]
        elif key_mode == KEY_ERASE_GATE:
            kw, kr, vw = k[t], be[t] * k[t], ga[t] * v[t]
        else:
            kw, kr, vw = be[t] * k[t], k[t], ga[t] * v[t]
        M = (torch.eye(dk, dtype=q.dtype) - torch.outer(kw, kr)) @ torch.diag(a)
        S = M @ S + torch.outer(kw, vw)
        outs.append(S.T @ q[t])
    return torch.stack(outs), S


@pytest.mark.parametrize("key_mode", [KEY_SYMMETRIC, KEY_ERASE_GATE, KEY_WRITE_GATE])
def test_bwd_matches_autograd_of_product_form(key_mode):
    """Reverse-mode autodiff (fp64) of the transition-product form agrees with the
    oracle's backward on every gradient (T = 48, dk = 8, dv = 6, vector gates)."""
    rng = np.random.default_rng(5)
    T, dk, dv = 48, 8, 6
    c = _case(rng, T=T, dk=dk, dv=dv, amode=ALPHA_VEC, bmode=GATE_VEC, gmode=GATE_VEC, precond=None)
    g = _grads(c, key_mode)
    names = ["q", "k", "v", "log_alpha", "beta", "gamma", "S0"]
    ts = {n: torch.tensor(c[n][0, 0], dtype=torch.float64, requires_grad=True) for n in names}
    o, ST = _torch_product_form(ts["q"], ts["k"], ts["v"], ts["log_alpha"], ts["beta"],
                                ts["gamma"], ts["S0"], key_mode)
    L = (o * torch.tensor(c["dO"][0, 0])).sum() + (ST * torch.tensor(c["dST"][0, 0])).sum()
    L.backward()
    for n, gn in zip(names, ["dq", "dk", "dv", "dlog_alpha", "dbeta", "dgamma", "dS0"]):
        np.testing.assert_allclose(g[gn][0, 0], ts[n].grad.numpy(), rtol=1e-10, atol=1e-11,
                                   err_msg=n)


def test_bwd_empty_sequence():
    """T = 0: dS0 = dST and every per-token gradient is empty."""
    rng = np.random.default_rng(1)
    c = _case(rng, T=0, dk=4, dv=3, amode=ALPHA_SCALAR, bmode=GATE_SCALAR, gmode=GATE_SCALAR,
              precond=PRECOND_INVERSE)
    g = _grads(c, KEY_SYMMETRIC)
    np.testing.assert_array_equal(g["dS0"], c["dST"])
    np.testing.assert_array_equal(g["dA0"], np.zeros_like(c["A0"]))
    assert g["dq"].shape == (1, 1, 0, 4)
