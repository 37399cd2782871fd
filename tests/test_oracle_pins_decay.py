"""Pins of the fp64 oracle's second rule (CPU only): the gated recurrence without the erase
term, S_t = a_t S_{t-1} + b_t v_t k_t^T, a_t = exp(g_t), o_t = S_t q_t / sqrt(d_k) -- the
uniform decay the Priming article (we0.ai, comparison of Mamba-2, Gated DeltaNet and Gated
KalmaNet) attributes to Mamba-2, set against GDN's key-selective erase.

Pinned to a hand-worked example, closed-form special cases, the explicit decayed-sum form
(a different algorithm from the recurrence) and the contrast with the delta rule.
"""
import json
import os

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DECAY = oracle.GATED_DECAY


def rand_inputs(B, T, H, dk, dv, seed, s0=True):
    d = gi.prefill_inputs(B, T, H, dk, dv, wid=901, call=seed, qkv_dtype=torch.float32, s0=s0)
    return {k: (None if x is None else x.to(torch.float64)) for k, x in d.items()}


def run(orc, d, rule=DECAY):
    return orc.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d.get("s0"), rule=rule)


def test_decay_hand_worked_example(orc):
    with open(os.path.join(GOLDEN, "hand_worked_decay_d2_t3.json")) as f:
        ex = json.load(f)
    arr = {k: np.array(ex[k], dtype=np.float64) for k in ("q", "k", "v", "g", "beta")}
    o, sf = orc.prefill(arr["q"], arr["k"], arr["v"], arr["g"], arr["beta"], rule=DECAY)
    np.testing.assert_allclose(o * np.sqrt(2.0), np.array(ex["o_times_sqrt2"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(sf, np.array(ex["final_state_key_major"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed,B,T,H,dk,dv,gate", [
    (1, 1, 9, 2, 4, 3, "primary"), (2, 2, 14, 1, 6, 2, "literal"), (3, 1, 7, 3, 3, 5, "primary")])
def test_decay_matches_explicit_decayed_sums(orc, seed, B, T, H, dk, dv, gate):
    d = rand_inputs(B, T, H, dk, dv, seed)
    if gate == "literal":
        d["g"] = -torch.nn.functional.softplus(torch.randn(B, T, H, dtype=torch.float64) + 3.0)
    d["beta"] = d["beta"] * 2.0  # b up to 2: no clamping anywhere
    o, sf = run(orc, d)
    eo, es = oracle.closed_form_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    scale = max(np.abs(eo).max(), 1e-300)
    assert np.abs(o - eo).max() <= 1e-12 * scale
    assert np.abs(sf - es).max() <= 1e-12 * max(np.abs(es).max(), 1e-300)


def test_decay_pure_decay_and_single_token(orc):
    d = rand_inputs(1, 23, 2, 5, 4, 4)
    d["beta"].zero_()
    o, sf = run(orc, d)
    G = np.cumsum(d["g"].numpy(), axis=1)
    s0 = d["s0"].numpy()
    np.testing.assert_allclose(sf, np.exp(G[:, -1])[:, :, None, None] * s0, rtol=1e-13, atol=0)
    # one token from a zero state: o = b (k . q) v / sqrt(d_k), as for the delta rule
    d = rand_inputs(2, 1, 3, 6, 4, 5, s0=False)
    o, _ = run(orc, d)
    q, k, v, b = (d[x].numpy() for x in ("q", "k", "v", "beta"))
    kq = np.einsum("bthj,bthj->bth", k, q)
    np.testing.assert_allclose(o, (b * kq)[..., None] * v / np.sqrt(6), rtol=1e-13, atol=1e-16)


def test_decay_accumulates_where_the_delta_rule_overwrites(orc):
    """a = 1, b = 1, one unit key written twice: the decay rule stores v1 + v2 under it, the
    delta rule only v2 (its erase removes v1 first)."""
    dk, dv = 4, 3
    k = np.zeros((1, 2, 1, dk)); k[0, :, 0, 1] = 1.0
    v = np.array([[[[1.0, -2.0, 0.5]], [[3.0, 1.0, -1.0]]]])
    q = k.copy()
    g = np.zeros((1, 2, 1)); b = np.ones((1, 2, 1))
    o_dec, s_dec = orc.prefill(q, k, v, g, b, rule=DECAY)
    o_del, s_del = orc.prefill(q, k, v, g, b, rule=oracle.GATED_DELTA)
    np.testing.assert_allclose(s_dec[0, 0, 1], v[0, 0, 0] + v[0, 1, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(s_del[0, 0, 1], v[0, 1, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o_dec[0, 1, 0] * 2.0, v[0, 0, 0] + v[0, 1, 0], rtol=0, atol=1e-15)


def test_decay_chaining_is_bitwise_and_decode_matches(orc):
    d = rand_inputs(2, 30, 2, 5, 3, 6)
    o, sf = run(orc, d)
    first = {k: (x if k == "s0" else x[:, :11]) for k, x in d.items()}
    o1, s1 = run(orc, first)
    rest = {k: (torch.from_numpy(s1) if k == "s0" else x[:, 11:]) for k, x in d.items()}
    o2, s2 = run(orc, rest)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o) and np.array_equal(s2, sf)
    state = d["s0"].numpy().copy()
    for t in range(30):
        od = orc.decode_step(d["q"][:, t], d["k"][:, t], d["v"][:, t], d["g"][:, t], d["beta"][:, t],
                             state, rule=DECAY)
        assert np.array_equal(od, o[:, t])
    assert np.array_equal(state, sf)


def test_rule_is_validated(orc):
    d = rand_inputs(1, 2, 1, 2, 2, 7)
    with pytest.raises(ValueError):
        run(orc, d, rule=7)
