"""Host checks of the seeded input generators (no GPU).

The generators hold no arithmetic of the method; these tests pin only what the
GPU tests and the oracle tests rely on: determinism in the seed, the stated
shapes, bf16-exact values where the GPU receives bf16, and that the streaming
form of the decode workload yields exactly the decode workload's steps.
"""
import numpy as np
import pytest

from gated_delta_rule_77_amd import synth


def test_decode_stream_matches_decode():
    w = synth.decode(B=3, H=2, d=16, steps=9, seed=5)
    S0, it = synth.decode_stream(B=3, H=2, d=16, steps=9, seed=5)
    assert np.array_equal(S0, w.S0)
    n = 0
    for t, (q, k, v, la, be, ga) in enumerate(it):
        for a, b in ((q, w.q), (k, w.k), (v, w.v), (la, w.log_alpha), (be, w.beta),
                     (ga, w.gamma)):
            assert np.array_equal(a, b[:, :, t]), t
        n += 1
    assert n == 9


@pytest.mark.parametrize("gen", ["deltanet_fp32", "gdn", "kda_fg2", "gdn2_precond"])
def test_generators_are_seeded_and_shaped(gen):
    kw = dict(B=1, H=2, T=70, d=64, seed=3)
    if gen == "gdn2_precond":
        kw["n_pairs"] = 4
    a, b = getattr(synth, gen)(**kw), getattr(synth, gen)(**kw)
    for name in ("q", "k", "v", "log_alpha", "beta", "gamma"):
        x, y = getattr(a, name), getattr(b, name)
        assert (x is None) == (y is None)
        if x is not None:
            assert np.array_equal(x, y)
            assert x.dtype == np.float32
    assert a.q.shape == (1, 2, 70, 64) and a.v.shape == (1, 2, 70, 64)
    if a.qkv_dtype == synth.DT_BF16:
        for x in (a.q, a.k, a.v):
            assert np.array_equal(synth.round_to_bf16(x), x)
    # unit-norm queries and keys (up to the bf16 rounding)
    assert np.allclose(np.linalg.norm(a.k.astype(np.float64), axis=-1), 1.0, atol=1e-2)


def test_round_to_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between two bf16 values: ties go to the even one (1)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0], np.float32)
    r = synth.round_to_bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0 + 2.0 ** -6 and r[2] == -2.5 and r[3] == 0.0
