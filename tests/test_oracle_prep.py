"""Pins of the input-preparation reference (CPU only): closed forms and invariants of each step."""
import numpy as np
import pytest

from oracle import prep

RNG = np.random.default_rng(3)


def raw(B=2, T=9, H=3, dk=4, dv=5):
    return (RNG.normal(size=(B, T, H, dk)), RNG.normal(size=(B, T, H, dk)), RNG.normal(size=(B, T, H, dv)),
            RNG.normal(size=(H * dk, 4)), RNG.normal(size=(H * dk, 4)), RNG.normal(size=(H * dv, 4)),
            RNG.normal(size=(B, T, H)) * 3, RNG.normal(size=(B, T, H)))


def test_identity_taps_pass_inputs_through():
    x = RNG.normal(size=(1, 7, 2, 3))
    w = np.tile([0.0, 0.0, 0.0, 1.0], (6, 1))
    c, st = prep.short_conv(x, w)
    assert np.array_equal(c, x)
    assert np.array_equal(st, np.transpose(x[0, 4:7].reshape(3, 6))[None])


def test_convolution_is_causal_and_matches_a_hand_sum():
    x = RNG.normal(size=(1, 6, 1, 2))
    w = RNG.normal(size=(2, 4))
    c, _ = prep.short_conv(x, w)
    # token 4, channel 1: w[1,0] x_1 + w[1,1] x_2 + w[1,2] x_3 + w[1,3] x_4
    hand = w[1, 0] * x[0, 1, 0, 1] + w[1, 1] * x[0, 2, 0, 1] + w[1, 2] * x[0, 3, 0, 1] + w[1, 3] * x[0, 4, 0, 1]
    assert abs(c[0, 4, 0, 1] - hand) < 1e-14
    # token 1 sees only x_0, x_1 (zero padding before the start)
    assert abs(c[0, 1, 0, 0] - (w[0, 2] * x[0, 0, 0, 0] + w[0, 3] * x[0, 1, 0, 0])) < 1e-14
    x2 = x.copy()
    x2[0, 5] += 1.0  # changing the last token changes nothing before it
    c2, _ = prep.short_conv(x2, w)
    assert np.array_equal(c2[0, :5], c[0, :5])


def test_carried_state_chains_calls_exactly():
    xq, xk, xv, wq, wk, wv, a, b = raw(T=11)
    whole = prep.prepare(xq, xk, xv, wq, wk, wv, a, b)
    first = prep.prepare(xq[:, :4], xk[:, :4], xv[:, :4], wq, wk, wv, a[:, :4], b[:, :4])
    rest = prep.prepare(xq[:, 4:], xk[:, 4:], xv[:, 4:], wq, wk, wv, a[:, 4:], b[:, 4:], first["conv_state"])
    for key in ("q", "k", "v", "g", "beta"):
        np.testing.assert_allclose(np.concatenate([first[key], rest[key]], axis=1), whole[key], rtol=0, atol=1e-15)
    np.testing.assert_allclose(rest["conv_state"], whole["conv_state"], rtol=0, atol=0)


def test_activation_norm_and_gates():
    assert prep.silu(np.array([0.0]))[0] == 0.0
    assert abs(prep.silu(np.array([2.0]))[0] - 2.0 / (1.0 + np.exp(-2.0))) < 1e-15
    xq, xk, xv, wq, wk, wv, a, b = raw()
    out = prep.prepare(xq, xk, xv, wq, wk, wv, a, b)
    n = np.sqrt(np.sum(out["q"] ** 2, axis=-1))
    y = prep.silu(prep.short_conv(xq, wq)[0])
    expect = np.sqrt(np.sum(y * y, axis=-1) / (np.sum(y * y, axis=-1) + prep.EPS))
    np.testing.assert_allclose(n, expect, rtol=1e-14)   # unit norm up to the epsilon
    assert np.all(out["g"] <= 0) and np.all((out["beta"] > 0) & (out["beta"] < 1))
    np.testing.assert_allclose(prep.prepare(xq, xk, xv, wq, wk, wv, np.zeros_like(a), np.zeros_like(b))["g"],
                               -np.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(prep.prepare(xq, xk, xv, wq, wk, wv, a, np.zeros_like(b))["beta"], 0.5, rtol=0)
    # v takes convolution and SiLU only (no norm)
    np.testing.assert_allclose(out["v"], prep.silu(prep.short_conv(xv, wv)[0]), rtol=0, atol=0)


def test_gate_rate_bias_and_known_values():
    xq, xk, xv, wq, wk, wv, a, b = raw(H=3)
    A = np.array([0.5, 1.0, 4.0])
    bias = np.array([0.25, -1.0, 2.0])
    out = prep.prepare(xq, xk, xv, wq, wk, wv, np.broadcast_to(-bias, a.shape), b, A=A, dt_bias=bias)
    np.testing.assert_allclose(out["g"], np.broadcast_to(-A * np.log(2.0), a.shape), rtol=1e-15)
    big = prep.prepare(xq, xk, xv, wq, wk, wv, np.full(a.shape, 800.0), b)  # softplus(z) = z for large z
    np.testing.assert_allclose(big["g"], -800.0, rtol=1e-15)
    tiny = prep.prepare(xq, xk, xv, wq, wk, wv, np.full(a.shape, -40.0), b)  # softplus(z) = e^z for z << 0
    np.testing.assert_allclose(tiny["g"], -np.exp(-40.0), rtol=1e-12)
    two = prep.prepare(xq, xk, xv, wq, wk, wv, a, np.full(b.shape, 2.0))
    np.testing.assert_allclose(two["beta"], 0.8807970779778823, rtol=1e-15)  # logistic(2)
    np.testing.assert_allclose(prep.silu(np.array([-1.0]))[0], -0.2689414213699951, rtol=1e-15)  # -logistic(-1)
