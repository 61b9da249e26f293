"""Pins for the fp64 oracle (CPU only).

The pages print no numeric example, so the oracle is pinned by what the
mathematics fixes: hand-derived worked examples (tests/golden), closed forms,
invariants, two independent formulations of the same recurrence
(explicit transition-matrix product; chunkwise UT/WY solve), and the special
cases the pages say the general rule reduces to.  Each test is chosen so that
a plausible slip in the oracle (a dropped term, a wrong sign, a transposed
operand, a decay applied after instead of before the erase, an exclusive
instead of inclusive preconditioner sum) fails at least one of them.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import (ALPHA_NONE, ALPHA_SCALAR, ALPHA_VEC, GATE_SCALAR, GATE_VEC,
                    GAMMA_SAME_AS_BETA, rel_l2)
from formulations import (apply_to_key_exact, apply_to_query_exact, axis_key_case, chunked_wy,
                          ridge_memory, unrolled_product)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.txt")


def _rand_case(rng, B, H, T, dk, dv, amode, bmode, gmode, precond=False, s0=True,
               a0=False):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    la = None
    if amode == ALPHA_SCALAR:
        la = -np.log1p(np.exp(rng.standard_normal((B, H, T))))
    elif amode == ALPHA_VEC:
        la = -np.log1p(np.exp(rng.standard_normal((B, H, T, dk))))
    if bmode == GATE_SCALAR:
        be = 1 / (1 + np.exp(-rng.standard_normal((B, H, T))))
    else:
        be = 1 / (1 + np.exp(-rng.standard_normal((B, H, T, dk))))
    ga = None
    if gmode == GATE_SCALAR:
        ga = 1 / (1 + np.exp(-rng.standard_normal((B, H, T))))
    elif gmode == GATE_VEC:
        ga = 1 / (1 + np.exp(-rng.standard_normal((B, H, T, dv))))
    S0 = 0.5 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    A0 = rng.uniform(0.5, 2.0, (B, H, dk)) if a0 else None
    return dict(q=q, k=k, v=v, alpha_mode=amode, log_alpha=la, beta_mode=bmode,
                beta=be, gamma_mode=gmode, gamma=ga,
                precond_eps=(1e-3 if precond else -1.0), A0=A0, S0=S0)


MODES = [
    (ALPHA_NONE, GATE_SCALAR, GAMMA_SAME_AS_BETA, False),   # DeltaNet
    (ALPHA_SCALAR, GATE_SCALAR, GAMMA_SAME_AS_BETA, False),  # Gated DeltaNet
    (ALPHA_VEC, GATE_SCALAR, GAMMA_SAME_AS_BETA, False),    # KDA
    (ALPHA_VEC, GATE_VEC, GAMMA_SAME_AS_BETA, False),       # FG^2-GDN
    (ALPHA_VEC, GATE_VEC, GATE_SCALAR, False),              # FG^2 key gain, scalar write
    (ALPHA_VEC, GATE_VEC, GATE_VEC, False),                 # GDN-2 style erase/write
    (ALPHA_SCALAR, GATE_SCALAR, GAMMA_SAME_AS_BETA, True),  # PGDN
    (ALPHA_VEC, GATE_VEC, GATE_VEC, True),                  # GDN-2 + preconditioner
]


def _parse_golden():
    blocks, cur = {}, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = blocks.setdefault(line.strip("[]"), {})
            continue
        key, val = [x.strip() for x in line.split("=", 1)]
        cur[key] = val
    return blocks


def _arr(s, width=None):
    toks = [np.array([float(x) for x in part.split()]) for part in s.split("|")]
    return np.stack(toks)


@pytest.mark.parametrize("name", ["example1", "example2"])
def test_worked_examples(name):
    ex = _parse_golden()[name]
    dk, dv = int(ex["dk"]), int(ex["dv"])
    k = _arr(ex["k"])[None, None]
    v = _arr(ex["v"])[None, None]
    q = _arr(ex["q"])[None, None]
    T = k.shape[2]
    amode = {"none": ALPHA_NONE, "scalar": ALPHA_SCALAR, "vec": ALPHA_VEC}[ex["alpha_mode"]]
    la = None
    if amode != ALPHA_NONE:
        la = _arr(ex["log_alpha"])
        if ex.get("log_alpha_is_exp") == "1":
            la = np.log(la)
        la = la[None, None] if amode == ALPHA_VEC else la[None, None, :, 0]
    bmode = {"scalar": GATE_SCALAR, "vec": GATE_VEC}[ex["beta_mode"]]
    be = _arr(ex["beta"])
    be = be[None, None, :, 0] if bmode == GATE_SCALAR else be[None, None]
    gmode = {"same": GAMMA_SAME_AS_BETA, "scalar": GATE_SCALAR, "vec": GATE_VEC}[ex["gamma_mode"]]
    ga = None
    if gmode != GAMMA_SAME_AS_BETA:
        ga = _arr(ex["gamma"])
        ga = ga[None, None, :, 0] if gmode == GATE_SCALAR else ga[None, None]
    eps = float(ex.get("precond_eps", -1))
    S0 = _arr(ex["S0"]).reshape(1, 1, dk, dv) if "S0" in ex else None
    o, ST, AT = oracle.delta_rule(q, k, v, amode, la, bmode, be, gmode, ga, eps, None, S0)
    np.testing.assert_allclose(o[0, 0], _arr(ex["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ST[0, 0].ravel(), _arr(ex["ST"]).ravel(), rtol=0, atol=1e-12)
    if "AT" in ex:
        np.testing.assert_allclose(AT[0, 0], _arr(ex["AT"]).ravel(), rtol=0, atol=1e-12)
    assert T == o.shape[2]


@pytest.mark.parametrize("amode,bmode,gmode,pre", MODES)
def test_matches_unrolled_transition_product(amode, bmode, gmode, pre):
    rng = np.random.default_rng(1)
    c = _rand_case(rng, 1, 2, 7, 4, 4, amode, bmode, gmode, pre, a0=pre)
    o, ST, _ = oracle.delta_rule(**c)
    o2, ST2 = unrolled_product(**c)
    np.testing.assert_allclose(o, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ST, ST2, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("amode,bmode,gmode,pre", MODES)
@pytest.mark.parametrize("T,C", [(37, 16), (64, 64), (5, 16)])
def test_matches_chunked_wy_form(amode, bmode, gmode, pre, T, C):
    rng = np.random.default_rng(2)
    dv = 8 if gmode != GAMMA_SAME_AS_BETA or bmode == GATE_SCALAR else 6
    c = _rand_case(rng, 2, 1, T, 6, dv, amode, bmode, gmode, pre)
    o, ST, _ = oracle.delta_rule(**c)
    o2, ST2 = chunked_wy(**c, C=C)
    assert rel_l2(o2, o) < 1e-11
    assert rel_l2(ST2, ST) < 1e-11


def test_c_oracle_matches_numpy_loop_layouts():
    # Same definition twice: checks the ctypes plumbing and memory layouts.
    rng = np.random.default_rng(3)
    for amode, bmode, gmode, pre in MODES:
        c = _rand_case(rng, 2, 3, 9, 5, 7 if gmode != GAMMA_SAME_AS_BETA or bmode == GATE_SCALAR else 5,
                       amode, bmode, gmode, pre, a0=pre)
        o, ST, AT = oracle.delta_rule(**c)
        o2, ST2, AT2 = oracle.delta_rule_py(**c)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ST, ST2, rtol=1e-12, atol=1e-13)
        if pre:
            np.testing.assert_allclose(AT, AT2, rtol=1e-13)


def test_zero_gain_only_decays():
    # beta = 0: nothing is erased or written; S_t = Diag(prod alpha) S_0 and
    # o_t = (Diag(Gamma_t) S_0)^T q_t with Gamma_t the cumulative decay.
    rng = np.random.default_rng(4)
    c = _rand_case(rng, 1, 2, 11, 5, 6, ALPHA_VEC, GATE_SCALAR, GATE_SCALAR)
    c["beta"] = np.zeros_like(c["beta"])
    o, ST, _ = oracle.delta_rule(**c)
    Gam = np.exp(np.cumsum(c["log_alpha"], axis=2))  # [B,H,T,dk]
    exp_o = np.einsum("bhti,bhij,bhti->bhtj", Gam, c["S0"], c["q"])
    np.testing.assert_allclose(o, exp_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ST, Gam[:, :, -1, :, None] * c["S0"], rtol=1e-12)
    # alpha == 1 as well: the state is untouched
    c["alpha_mode"], c["log_alpha"] = ALPHA_NONE, None
    o, ST, _ = oracle.delta_rule(**c)
    np.testing.assert_array_equal(ST, c["S0"])


def test_exact_retrieval_with_orthonormal_keys():
    # alpha = 1, beta = gamma = 1, orthonormal keys: after writing every key
    # once, S^T k_i = v_i for all i (each write fully replaces its slot and
    # leaves the orthogonal directions alone).
    rng = np.random.default_rng(5)
    d = 8
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T[None, None]                  # rows are orthonormal keys
    v = rng.standard_normal((1, 1, d, d))
    S0 = rng.standard_normal((1, 1, d, d))
    o, ST, _ = oracle.delta_rule(k.copy(), k, v, ALPHA_NONE, None, GATE_SCALAR,
                                 np.ones((1, 1, d)), GAMMA_SAME_AS_BETA, None, S0=S0)
    np.testing.assert_allclose(ST[0, 0].T @ k[0, 0].T, v[0, 0].T, atol=1e-12)
    # querying with the key just written returns its value at that step
    np.testing.assert_allclose(o[0, 0], v[0, 0], atol=1e-12)


def test_overwrite_same_key():
    # A unit key written twice with beta = 1 holds only the second value.
    rng = np.random.default_rng(6)
    d = 6
    kk = rng.standard_normal(d)
    kk /= np.linalg.norm(kk)
    k = np.stack([kk, kk])[None, None]
    v = rng.standard_normal((1, 1, 2, d))
    o, ST, _ = oracle.delta_rule(k.copy(), k, v, ALPHA_NONE, None, GATE_SCALAR,
                                 np.ones((1, 1, 2)), GAMMA_SAME_AS_BETA, None,
                                 S0=rng.standard_normal((1, 1, d, d)))
    np.testing.assert_allclose(ST[0, 0].T @ kk, v[0, 0, 1], atol=1e-12)


def test_register_file_semantics_exact():
    # One-hot keys and queries, alpha = 1, beta in {0, 1}, integer values:
    # the state acts as a register file (beta=1 overwrites row j, beta=0 is a
    # no-op) and every quantity stays an integer, so the comparison is exact.
    rng = np.random.default_rng(7)
    dk, dv, T = 8, 5, 200
    kj = rng.integers(0, dk, T)
    qj = rng.integers(0, dk, T)
    gate = rng.integers(0, 2, T).astype(np.float64)
    v = rng.integers(-8, 9, (T, dv)).astype(np.float64)
    S0 = rng.integers(-8, 9, (dk, dv)).astype(np.float64)
    k = np.eye(dk)[kj]
    q = np.eye(dk)[qj]
    o, ST, _ = oracle.delta_rule(q[None, None], k[None, None], v[None, None], ALPHA_NONE,
                                 None, GATE_SCALAR, gate[None, None], GAMMA_SAME_AS_BETA,
                                 None, S0=S0[None, None])
    mem = S0.copy()
    exp_o = np.zeros((T, dv))
    for t in range(T):
        if gate[t] == 1:
            mem[kj[t]] = v[t]
        exp_o[t] = mem[qj[t]]
    np.testing.assert_array_equal(o[0, 0], exp_o)
    np.testing.assert_array_equal(ST[0, 0], mem)


def test_linearity():
    # o is linear in (S_0, v) jointly and linear in q (gates held fixed).
    rng = np.random.default_rng(8)
    c1 = _rand_case(rng, 1, 1, 13, 5, 5, ALPHA_VEC, GATE_VEC, GATE_VEC)
    c2 = dict(c1)
    c2["v"] = rng.standard_normal(c1["v"].shape)
    c2["S0"] = rng.standard_normal(c1["S0"].shape)
    a, b = 0.7, -1.3
    c3 = dict(c1)
    c3["v"] = a * c1["v"] + b * c2["v"]
    c3["S0"] = a * c1["S0"] + b * c2["S0"]
    o1, S1, _ = oracle.delta_rule(**c1)
    o2, S2, _ = oracle.delta_rule(**c2)
    o3, S3, _ = oracle.delta_rule(**c3)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S3, a * S1 + b * S2, rtol=1e-11, atol=1e-12)
    c4 = dict(c1)
    c4["q"] = 2.0 * c1["q"]
    o4, _, _ = oracle.delta_rule(**c4)
    np.testing.assert_allclose(o4, 2.0 * o1, rtol=1e-13)


def test_preconditioner_closed_form_one_hot():
    # One-hot keys e_j, beta = 1, gamma scalar g, alpha = 1: the key Gram
    # diagonal counts writes, so the n-th write to row j uses
    # c_n = 1 / (A0_j + n + eps) and gives S_j <- (1 - c_n) S_j + sqrt(c_n g) v.
    rng = np.random.default_rng(9)
    dk, dv, T, eps = 4, 3, 40, 1e-6
    kj = rng.integers(0, dk, T)
    k = np.eye(dk)[kj]
    v = rng.standard_normal((T, dv))
    g = rng.uniform(0.2, 1.0, T)
    A0 = rng.uniform(0.0, 3.0, dk)
    o, ST, AT = oracle.delta_rule(k[None, None], k[None, None], v[None, None], ALPHA_NONE,
                                  None, GATE_SCALAR, np.ones((1, 1, T)), GATE_SCALAR,
                                  g[None, None], eps, A0[None, None], None)
    mem = np.zeros((dk, dv))
    cnt = A0.copy()
    for t in range(T):
        j = kj[t]
        cnt[j] += 1.0
        c = 1.0 / (cnt[j] + eps)
        mem[j] = (1 - c) * mem[j] + np.sqrt(c * g[t]) * v[t]
    np.testing.assert_allclose(ST[0, 0], mem, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(AT[0, 0], cnt, rtol=0, atol=0)


def test_preconditioner_accumulator_is_exact_sum():
    # A_T = A_0 + sum_t k_t (.) k_t for bf16-valued keys (exact in fp64).
    from gated_delta_rule_77_amd import synth
    w = synth.gdn2_precond(B=1, H=2, T=300, d=16, n_pairs=8)
    A0 = np.arange(32, dtype=np.float64).reshape(1, 2, 16) / 8
    _, _, AT = oracle.delta_rule(w.q, w.k, w.v, w.alpha_mode, w.log_alpha, w.beta_mode,
                                 w.beta, w.gamma_mode, w.gamma, w.precond_eps, A0, None)
    k = w.k.astype(np.float64)
    np.testing.assert_array_equal(AT, A0 + np.sum(k * k, axis=2))


@pytest.mark.parametrize("which", ["beta_vec_equal", "alpha_vec_equal", "gamma_same"])
def test_mode_reductions(which):
    # Gated DeltaNet-2 reduces to KDA when erase and write gates are tied to
    # one scalar, and to Gated DeltaNet when the decay is scalar too; a vector
    # gate with equal entries must equal the scalar path exactly.
    rng = np.random.default_rng(10)
    B, H, T, d = 1, 2, 20, 6
    c = _rand_case(rng, B, H, T, d, d, ALPHA_SCALAR, GATE_SCALAR, GAMMA_SAME_AS_BETA)
    o_ref, S_ref, _ = oracle.delta_rule(**c)
    c2 = dict(c)
    if which == "beta_vec_equal":
        c2["beta_mode"] = GATE_VEC
        c2["beta"] = np.repeat(c["beta"][..., None], d, axis=-1)
    elif which == "alpha_vec_equal":
        c2["alpha_mode"] = ALPHA_VEC
        c2["log_alpha"] = np.repeat(c["log_alpha"][..., None], d, axis=-1)
    else:
        c2["gamma_mode"] = GATE_SCALAR
        c2["gamma"] = c["beta"].copy()
    o2, S2, _ = oracle.delta_rule(**c2)
    np.testing.assert_allclose(o2, o_ref, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S2, S_ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("pre", [False, True])
def test_split_call_continuation(pre):
    # fwd(x[0:T]) == fwd(x[t0:T], S0 = S_T(x[0:t0]), A0 = A_T(x[0:t0]))
    rng = np.random.default_rng(11)
    c = _rand_case(rng, 1, 2, 30, 5, 5, ALPHA_VEC, GATE_VEC, GATE_VEC, pre, a0=pre)
    o, ST, AT = oracle.delta_rule(**c)
    t0 = 13
    sl = lambda x, a, b: None if x is None else x[:, :, a:b]
    ca = dict(c, q=sl(c["q"], 0, t0), k=sl(c["k"], 0, t0), v=sl(c["v"], 0, t0),
              log_alpha=sl(c["log_alpha"], 0, t0), beta=sl(c["beta"], 0, t0),
              gamma=sl(c["gamma"], 0, t0))
    oa, Sa, Aa = oracle.delta_rule(**ca)
    cb = dict(c, q=sl(c["q"], t0, 30), k=sl(c["k"], t0, 30), v=sl(c["v"], t0, 30),
              log_alpha=sl(c["log_alpha"], t0, 30), beta=sl(c["beta"], t0, 30),
              gamma=sl(c["gamma"], t0, 30), S0=Sa, A0=Aa)
    ob, Sb, Ab = oracle.delta_rule(**cb)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=2), o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Sb, ST, rtol=1e-12, atol=1e-14)
    if pre:
        np.testing.assert_allclose(Ab, AT, rtol=1e-14)


def test_contraction_bound():
    # ||kt|| <= 1 and alpha <= 1 make (I - kt kt^T) Diag(alpha) non-expansive,
    # so ||S_t||_F <= ||S_{t-1}||_F + ||kt|| ||vt||  (stability of the
    # transition, eigenvalues in the unit disc).
    rng = np.random.default_rng(12)
    c = _rand_case(rng, 1, 1, 50, 6, 6, ALPHA_VEC, GATE_VEC, GATE_VEC)
    prev = np.linalg.norm(c["S0"])
    for t in range(1, 50):
        ct = dict(c, q=c["q"][:, :, :t], k=c["k"][:, :, :t], v=c["v"][:, :, :t],
                  log_alpha=c["log_alpha"][:, :, :t], beta=c["beta"][:, :, :t],
                  gamma=c["gamma"][:, :, :t])
        _, St, _ = oracle.delta_rule(**ct)
        cur = np.linalg.norm(St)
        kt = np.sqrt(c["beta"][0, 0, t - 1]) * c["k"][0, 0, t - 1]
        vt = np.sqrt(c["gamma"][0, 0, t - 1]) * c["v"][0, 0, t - 1]
        assert cur <= prev + np.linalg.norm(kt) * np.linalg.norm(vt) + 1e-12
        prev = cur


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(13)
    c = _rand_case(rng, 1, 2, 0, 4, 4, ALPHA_VEC, GATE_VEC, GATE_VEC, True, a0=True)
    o, ST, AT = oracle.delta_rule(**c)
    assert o.shape == (1, 2, 0, 4)
    np.testing.assert_array_equal(ST, c["S0"])
    np.testing.assert_array_equal(AT, c["A0"])


def test_planted_pairs_are_recalled_without_decay():
    # Sanity of the NIAH-shaped workload: with no decay and beta = gamma = 1 on
    # orthonormal planted keys only, the final queries return the planted values.
    from gated_delta_rule_77_amd import synth
    w = synth.gdn2_precond(B=1, H=1, T=256, d=32, n_pairs=8)
    pos, perm = w.meta["positions"][0, 0], w.meta["perms"][0, 0]
    T = w.T
    assert np.array_equal(w.q[0, 0, T - 8:], w.k[0, 0, pos][perm])
    assert np.array_equal(w.v[0, 0, pos][perm], w.v[0, 0, pos[perm]])


# ---------------------------------------------------------------------------
# read / write key modes: Gated DeltaNet-2's erase gate (method 1) and
# Preconditioned DeltaNet's apply-to-key write key
# ---------------------------------------------------------------------------

KEY_MODES = [oracle.KEY_ERASE_GATE, oracle.KEY_WRITE_GATE]
ASYM_GATES = [
    (ALPHA_VEC, GATE_VEC, GATE_VEC, False),
    (ALPHA_VEC, GATE_VEC, GAMMA_SAME_AS_BETA, True),
    (ALPHA_SCALAR, GATE_SCALAR, GATE_SCALAR, True),
    (ALPHA_NONE, GATE_VEC, GATE_SCALAR, False),
]


@pytest.mark.parametrize("key_mode", KEY_MODES)
@pytest.mark.parametrize("amode", [ALPHA_NONE, ALPHA_SCALAR, ALPHA_VEC])
def test_key_modes_reduce_to_tied_scalar_gain(key_mode, amode):
    # With one scalar gain per token serving as erase gate, write gate and
    # key gain, the erase-gate and apply-to-key updates are both
    # (I - beta k k^T) D S + beta k v^T: the symmetric form (Gated DeltaNet /
    # KDA), which the pins above fix.
    rng = np.random.default_rng(40)
    c = _rand_case(rng, 1, 2, 23, 6, 5, amode, GATE_SCALAR, GAMMA_SAME_AS_BETA)
    o_ref, S_ref, _ = oracle.delta_rule(**c)
    o, S, _ = oracle.delta_rule(**c, key_mode=key_mode)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("key_mode", KEY_MODES)
@pytest.mark.parametrize("gmode", [GAMMA_SAME_AS_BETA, GATE_VEC])
def test_key_modes_read_back_the_written_value(key_mode, gmode):
    # The fast-weight view of the update ("Gated DeltaNet-2" method 2): one
    # step edits the memory so that reading it with the read key returns the
    # gated target, whenever write key . read key = 1.  The read key is
    # e = b (.) k for the erase gate and the plain key for apply-to-key
    # (whose write key carries the gain); the target is w (.) v for the erase
    # gate, and v (or gamma (.) v) for apply-to-key.  Reading with the other
    # key does not return it, so a swap of the two keys fails here.
    rng = np.random.default_rng(41)
    dk = 5
    dv = dk if gmode == GAMMA_SAME_AS_BETA else 4   # a vector gain read as gamma needs dk == dv
    k = rng.standard_normal(dk)
    b = rng.uniform(0.2, 0.9, dk)
    k /= np.sqrt(np.sum(b * k * k))           # b (.) k . k = 1
    v = rng.standard_normal(dv)
    g = rng.uniform(0.2, 0.9, dv) if gmode == GATE_VEC else None
    S0 = rng.standard_normal((dk, dv))
    la = -rng.uniform(0.05, 0.5, dk)
    o, S, _ = oracle.delta_rule(np.zeros((1, 1, 1, dk)), k[None, None, None], v[None, None, None],
                                ALPHA_VEC, la[None, None, None], GATE_VEC, b[None, None, None],
                                gmode, None if g is None else g[None, None, None],
                                S0=S0[None, None], key_mode=key_mode)
    S = S[0, 0]
    if key_mode == oracle.KEY_ERASE_GATE:
        read, other = b * k, k
        target = (b if gmode == GAMMA_SAME_AS_BETA else g) * v
    else:
        read, other = k, b * k
        target = v if gmode == GAMMA_SAME_AS_BETA else g * v
    np.testing.assert_allclose(S.T @ read, target, rtol=1e-12, atol=1e-12)
    assert np.linalg.norm(S.T @ other - target) > 1e-3


@pytest.mark.parametrize("key_mode", KEY_MODES)
@pytest.mark.parametrize("amode,bmode,gmode,pre", ASYM_GATES)
def test_key_modes_match_unrolled_transition_product(key_mode, amode, bmode, gmode, pre):
    rng = np.random.default_rng(42)
    dv = 4 if not (gmode == GAMMA_SAME_AS_BETA and bmode == GATE_VEC) else 5
    c = _rand_case(rng, 1, 2, 7, 5, dv, amode, bmode, gmode, pre, a0=pre)
    o, ST, _ = oracle.delta_rule(**c, key_mode=key_mode)
    o2, ST2 = unrolled_product(**c, key_mode=key_mode)
    np.testing.assert_allclose(o, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ST, ST2, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("key_mode", KEY_MODES)
@pytest.mark.parametrize("amode,bmode,gmode,pre", ASYM_GATES)
@pytest.mark.parametrize("T,C", [(37, 16), (5, 16)])
def test_key_modes_match_chunked_wy_form(key_mode, amode, bmode, gmode, pre, T, C):
    rng = np.random.default_rng(43)
    dv = 8 if not (gmode == GAMMA_SAME_AS_BETA and bmode == GATE_VEC) else 6
    c = _rand_case(rng, 2, 1, T, 6, dv, amode, bmode, gmode, pre)
    o, ST, _ = oracle.delta_rule(**c, key_mode=key_mode)
    o2, ST2 = chunked_wy(**c, C=C, key_mode=key_mode)
    assert rel_l2(o2, o) < 1e-11
    assert rel_l2(ST2, ST) < 1e-11


@pytest.mark.parametrize("key_mode", KEY_MODES)
def test_key_modes_c_oracle_matches_numpy_loop(key_mode):
    rng = np.random.default_rng(44)
    c = _rand_case(rng, 2, 2, 9, 4, 4, ALPHA_VEC, GATE_VEC, GATE_VEC, True, a0=True)
    o, ST, AT = oracle.delta_rule(**c, key_mode=key_mode)
    o2, ST2, AT2 = oracle.delta_rule_py(**c, key_mode=key_mode)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ST, ST2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(AT, AT2, rtol=1e-12, atol=1e-14)


def test_key_modes_differ_with_vector_gains():
    # with a per-channel gain the three modes are three different recurrences
    rng = np.random.default_rng(45)
    c = _rand_case(rng, 1, 1, 12, 5, 5, ALPHA_VEC, GATE_VEC, GATE_VEC)
    outs = [oracle.delta_rule(**c, key_mode=m)[0] for m in
            (oracle.KEY_SYMMETRIC, oracle.KEY_ERASE_GATE, oracle.KEY_WRITE_GATE)]
    for i in range(3):
        for j in range(i + 1, 3):
            assert rel_l2(outs[i], outs[j]) > 1e-3


# ---------------------------------------------------------------------------
# exact preconditioner ("Preconditioned DeltaNet", Theorem 3.1)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lam", [1e-3, 1.0])
def test_exact_preconditioner_atk_atq_and_least_squares_agree(lam):
    # With the inverse (ridge) Gram matrix as preconditioner, DeltaNet on the
    # write key and linear attention on the query both return the
    # least-squares memory's prediction at every step.
    rng = np.random.default_rng(61)
    T, dk, dv = 40, 8, 5
    q, k, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    ridge = ridge_memory(k, v, lam)
    o_ref = np.einsum("tkv,tk->tv", ridge, q)
    o_atk, S_atk = apply_to_key_exact(q, k, v, lam)
    o_atq = apply_to_query_exact(q, k, v, lam)
    np.testing.assert_allclose(o_atk, o_ref, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(o_atq, o_ref, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(S_atk, ridge[-1], rtol=1e-9, atol=1e-11)


def test_exact_preconditioner_reaches_unregularised_least_squares():
    # once t >= dk the keys span the space and the vanishing-ridge memory is
    # the ordinary least-squares solution (numpy's lstsq, an independent routine)
    rng = np.random.default_rng(62)
    T, dk, dv = 30, 6, 4
    q, k, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    o_atk, _ = apply_to_key_exact(q, k, v, 1e-10)
    for t in range(dk, T):
        S_ls = np.linalg.lstsq(k[:t + 1], v[:t + 1], rcond=None)[0]
        np.testing.assert_allclose(o_atk[t], S_ls.T @ q[t], rtol=1e-6, atol=1e-8)


def test_first_order_delta_rule_is_not_least_squares():
    # the plain delta rule (unit gain, no preconditioner) is a gradient step,
    # not the least-squares solution: the references must tell them apart
    rng = np.random.default_rng(63)
    T, dk, dv = 30, 6, 4
    q, k, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    o_ls = np.einsum("tkv,tk->tv", ridge_memory(k, v, 1e-10), q)
    o_dn, _, _ = oracle.delta_rule(q[None, None], k[None, None], v[None, None], ALPHA_NONE, None,
                                   GATE_SCALAR, np.ones((1, 1, T)), GAMMA_SAME_AS_BETA, None)
    assert np.abs(o_dn[0, 0, dk:] - o_ls[dk:]).max() > 1e-2


@pytest.mark.parametrize("eps", [1e-3, 0.5])
def test_diagonal_preconditioner_is_exact_for_axis_keys(eps):
    # For keys along coordinate axes the running k (.) k sum is the whole Gram
    # matrix, so the diagonal preconditioner 1/(A_t + eps) on the write key
    # (write-gate mode, unit gain, no decay) is the exact ridge preconditioner
    # with lam = eps: the oracle must return the ridge memory.
    rng = np.random.default_rng(64)
    T, dk, dv = 50, 10, 6
    q, k, v = axis_key_case(rng, T, dk, dv, n_axes=7)
    o, S, _ = oracle.delta_rule(q[None, None], k[None, None], v[None, None], ALPHA_NONE, None,
                                GATE_SCALAR, np.ones((1, 1, T)), GAMMA_SAME_AS_BETA, None,
                                precond_eps=eps, key_mode=oracle.KEY_WRITE_GATE)
    ridge = ridge_memory(k, v, eps)
    np.testing.assert_allclose(o[0, 0], np.einsum("tkv,tk->tv", ridge, q), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], ridge[-1], rtol=1e-10, atol=1e-12)
    # the erase-gate and symmetric forms are not the exact preconditioner
    o_e, _, _ = oracle.delta_rule(q[None, None], k[None, None], v[None, None], ALPHA_NONE, None,
                                  GATE_SCALAR, np.ones((1, 1, T)), GAMMA_SAME_AS_BETA, None,
                                  precond_eps=eps, key_mode=oracle.KEY_SYMMETRIC)
    assert np.abs(o_e[0, 0] - np.einsum("tkv,tk->tv", ridge, q)).max() > 1e-3


# ---------------------------------------------------------------------------
# stabilised preconditioner (the reading of "Preconditioned DeltaNet" Eq. 9:
# B = x^-(r / (1 + |r|)), r = ln(A + eps) - mean over channels).  These pin the
# reading; its parity with the pages' own formula is unpinned.
# ---------------------------------------------------------------------------

def _no_precond(c):
    c.pop("precond_eps")
    c.pop("A0")
    return c


def _coeff_from_one_token(A, eps, x, beta=0.64, gamma=0.81):
    """Run the C oracle for one token from a zero state with k = sqrt(A)
    (so the running sum is A) and read the coefficient back from
    S_1 = sqrt(beta B) k (sqrt(gamma) v)^T."""
    dk = len(A)
    k = np.sqrt(np.asarray(A, np.float64))
    v = np.linspace(0.5, 1.5, 3)
    q = np.ones(dk)
    _, S, _ = oracle.delta_rule(q[None, None, None], k[None, None, None], v[None, None, None],
                                ALPHA_NONE, None, GATE_SCALAR, np.full((1, 1, 1), beta),
                                GATE_SCALAR, np.full((1, 1, 1), gamma), precond_eps=eps,
                                precond_mode=oracle.PRECOND_STABILISED, precond_x=x)
    return (S[0, 0] / (k[:, None] * np.sqrt(gamma) * v[None, :])) ** 2 / beta


def test_stabilised_coefficient_closed_form():
    # ln A = (1, -1): mean 0, r = (1, -1), s = (1/2, -1/2), B = (x^-1/2, x^1/2);
    # ln A = (2, 0, 0, -2): s = (2/3, 0, 0, -2/3)
    x, eps = 1.5, 0.0
    B = _coeff_from_one_token([np.e, np.exp(-1.0)], eps, x)
    np.testing.assert_allclose(B, np.repeat([[x ** -0.5], [x ** 0.5]], 3, axis=1), rtol=1e-12)
    B = _coeff_from_one_token([np.exp(2.0), 1.0, 1.0, np.exp(-2.0)], eps, x)
    want = np.array([x ** (-2 / 3), 1.0, 1.0, x ** (2 / 3)])
    np.testing.assert_allclose(B, np.repeat(want[:, None], 3, axis=1), rtol=1e-12)
    # eps enters inside the logarithm
    B = _coeff_from_one_token([np.e - 0.25, np.exp(-1.0) - 0.25], 0.25, 2.0)
    np.testing.assert_allclose(B[:, 0], [2.0 ** -0.5, 2.0 ** 0.5], rtol=1e-12)


@pytest.mark.parametrize("x", [1.2, 1.5, 2.0])
def test_stabilised_coefficient_bounds_and_scale_invariance(x):
    rng = np.random.default_rng(71)
    A = np.exp(rng.normal(0.0, 4.0, 16))  # heavy-tailed second moments
    B = _coeff_from_one_token(A, 0.0, x)[:, 0]
    assert np.all(B > 1.0 / x) and np.all(B < x)
    # larger second moment, smaller coefficient
    order = np.argsort(A)
    assert np.all(np.diff(B[order]) <= 1e-12)
    # scaling every key by c shifts ln A by 2 ln c: the centred r, hence B, is unchanged
    np.testing.assert_allclose(_coeff_from_one_token(A * 9.0, 0.0, x)[:, 0], B, rtol=1e-10)
    np.testing.assert_allclose(oracle.precond_coeff(A, 0.0, oracle.PRECOND_STABILISED, x), B,
                               rtol=1e-10)


def test_stabilised_is_identity_for_equal_channel_moments():
    # keys whose entries have equal magnitude in every channel give equal
    # running sums, so r = 0 and B = 1: the recurrence is the one without a
    # preconditioner, for every gate mode
    rng = np.random.default_rng(72)
    B_, H, T, dk, dv = 1, 2, 40, 8, 5
    c = _no_precond(_rand_case(rng, B_, H, T, dk, dv, ALPHA_VEC, GATE_VEC, GATE_VEC))
    c["k"] = rng.choice([-1.0, 1.0], (B_, H, T, dk)) / np.sqrt(dk)
    plain = oracle.delta_rule(**c)
    stab = oracle.delta_rule(**c, precond_eps=0.0, precond_mode=oracle.PRECOND_STABILISED,
                             precond_x=1.5)
    np.testing.assert_allclose(stab[0], plain[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(stab[1], plain[1], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("key_mode", KEY_MODES)
def test_stabilised_c_matches_numpy_loop_and_chunked_form(key_mode):
    rng = np.random.default_rng(73)
    c = _no_precond(_rand_case(rng, 1, 2, 37, 6, 4, ALPHA_VEC, GATE_VEC, GATE_SCALAR))
    A0 = rng.uniform(0.0, 1.0, (1, 2, 6))
    kw = dict(precond_eps=1e-3, A0=A0, precond_mode=oracle.PRECOND_STABILISED, precond_x=1.5,
              key_mode=key_mode)
    o, S, AT = oracle.delta_rule(**c, **kw)
    o2, S2, AT2 = oracle.delta_rule_py(**c, **kw)
    np.testing.assert_allclose(o, o2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S, S2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(AT, AT2, rtol=1e-13)
    o3, S3 = chunked_wy(**c, **kw, C=8)
    np.testing.assert_allclose(o, o3, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(S, S3, rtol=1e-9, atol=1e-11)


def test_stabilised_differs_from_inverse_and_rejects_bad_x():
    rng = np.random.default_rng(74)
    c = _no_precond(_rand_case(rng, 1, 1, 20, 6, 4, ALPHA_SCALAR, GATE_SCALAR, GAMMA_SAME_AS_BETA))
    inv = oracle.delta_rule(**c, precond_eps=1e-6)
    stab = oracle.delta_rule(**c, precond_eps=1e-6, precond_mode=oracle.PRECOND_STABILISED,
                             precond_x=1.5)
    assert np.abs(inv[0] - stab[0]).max() > 1e-3
    np.testing.assert_array_equal(inv[2], stab[2])  # the running sum itself is the same
    with pytest.raises(ValueError):
        oracle.delta_rule(**c, precond_eps=1e-6, precond_mode=oracle.PRECOND_STABILISED,
                          precond_x=1.0)
