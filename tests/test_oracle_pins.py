"""Pins of the fp64 oracle against facts fixed by the rule itself (CPU only).

The pages describe the GDN layer in words only (kwkr.cn digest of
HyLo-Llama-8MLA8GDN-8K-SFT, architecture section: gated delta-rule linear
attention with a fixed-size recurrent state; we0.ai Priming article, SSM
comparison: erases or rewrites the value held under one key) and print no
numeric example, so the oracle is pinned to closed forms, special cases,
invariants, a hand-worked example and an independent brute-force evaluation
of the same rule:

    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  a_t = exp(g_t),
    o_t = S_t q_t / sqrt(d_k);  states stored key-major [.., d_k, d_v].
"""
import json
import os

import numpy as np
import pytest
import torch

import gdn_inputs as gi

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(B, T, H, dk, dv, seed, s0=True, dtype=torch.float64):
    d = gi.prefill_inputs(B, T, H, dk, dv, wid=900, call=seed, qkv_dtype=torch.float32, s0=s0)
    return {k: (None if x is None else x.to(dtype)) for k, x in d.items()}


def run(orc, d, **kw):
    return orc.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d.get("s0"), **kw)


# --- hand-worked example -------------------------------------------------------------

def test_hand_worked_example(orc):
    with open(os.path.join(GOLDEN, "hand_worked_d2_t3.json")) as f:
        ex = json.load(f)
    arr = {k: np.array(ex[k], dtype=np.float64) for k in ("q", "k", "v", "g", "beta")}
    o, sf = orc.prefill(arr["q"], arr["k"], arr["v"], arr["g"], arr["beta"])
    np.testing.assert_allclose(o * np.sqrt(2.0), np.array(ex["o_times_sqrt2"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(sf, np.array(ex["final_state_key_major"]), rtol=0, atol=1e-14)


# --- closed forms of special cases ---------------------------------------------------------

def test_p1_identity_when_no_write_and_no_decay(orc):
    """b = 0, a = 1: the state never changes and o_t = S0 q_t / sqrt(d_k)."""
    d = rand_inputs(2, 19, 3, 8, 5, 1)
    d["beta"].zero_()
    d["g"].zero_()
    o, sf = run(orc, d)
    s0 = d["s0"].numpy()
    assert np.array_equal(sf, s0)
    expect = np.einsum("bthj,bhji->bthi", d["q"].numpy(), s0) / np.sqrt(8)
    np.testing.assert_allclose(o, expect, rtol=0, atol=1e-14)


def test_p2_pure_decay(orc):
    """b = 0: S_t = exp(sum_{i<=t} g_i) S0, in and across any chunking."""
    d = rand_inputs(1, 40, 2, 6, 4, 2)
    d["beta"].zero_()
    o, sf = run(orc, d)
    G = np.cumsum(d["g"].numpy(), axis=1)  # [B,T,H]
    s0 = d["s0"].numpy()
    np.testing.assert_allclose(sf, np.exp(G[:, -1])[:, :, None, None] * s0, rtol=1e-13, atol=0)
    expect = np.exp(G)[..., None] * np.einsum("bthj,bhji->bthi", d["q"].numpy(), s0) / np.sqrt(6)
    np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-15)


def test_p3_zero_gate_resets_to_rank_one(orc):
    """a = 0 (g = -inf): S_t = b_t v_t k_t^T and o_t = b_t (k_t . q_t) v_t / sqrt(d_k)."""
    d = rand_inputs(2, 9, 2, 7, 3, 3)
    d["g"].fill_(-np.inf)
    o, sf = run(orc, d)
    q, k, v, b = (d[x].numpy() for x in ("q", "k", "v", "beta"))
    kq = np.einsum("bthj,bthj->bth", k, q)
    np.testing.assert_allclose(o, (b * kq)[..., None] * v / np.sqrt(7), rtol=1e-13, atol=1e-16)
    last = b[:, -1, :, None, None] * np.einsum("bhj,bhi->bhji", k[:, -1], v[:, -1])
    np.testing.assert_allclose(sf, last, rtol=1e-13, atol=1e-16)


def test_p4_orthonormal_keys_exact_retrieval_and_overwrite(orc):
    """b = 1, a = 1, orthonormal keys: S k_j returns the latest value written under k_j."""
    rng = np.random.default_rng(4)
    dk, dv, m = 8, 5, 6
    Kq, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Kq[:, :m].T  # m orthonormal keys
    vals = rng.standard_normal((m, dv))
    newv = rng.standard_normal(dv)
    # write all m keys, then rewrite key 2 with a new value
    k = np.concatenate([keys, keys[2:3]])[None, :, None, :]
    v = np.concatenate([vals, newv[None]])[None, :, None, :]
    T = k.shape[1]
    q = np.zeros_like(k)
    g = np.zeros((1, T, 1))
    b = np.ones((1, T, 1))
    _, sf = orc.prefill(q, k, v, g, b)
    S = sf[0, 0].T  # [dv, dk]
    got = keys @ S.T  # row j = S k_j
    expect = vals.copy()
    expect[2] = newv
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-13)
    # from an arbitrary start state, one b=1 write of (k, v) makes S k = v exactly
    s0 = rng.standard_normal((1, 1, dk, dv))
    _, sf = orc.prefill(q[:, :1], k[:, :1], v[:, :1], g[:, :1], b[:, :1], s0)
    np.testing.assert_allclose(sf[0, 0].T @ keys[0], vals[0], rtol=0, atol=1e-13)


def test_p5_single_token_from_zero_state(orc):
    """One token from zeros: o = b (k . q) v / sqrt(d_k) -- the readout sees S_t, not S_{t-1}."""
    d = rand_inputs(3, 1, 4, 16, 16, 5, s0=False)
    o, _ = run(orc, d)
    q, k, v, b = (d[x].numpy() for x in ("q", "k", "v", "beta"))
    expect = (b * np.einsum("bthj,bthj->bth", k, q))[..., None] * v / 4.0
    np.testing.assert_allclose(o, expect, rtol=1e-14, atol=1e-17)


def test_p11_householder_reflection_preserves_norm(orc):
    """b = 2, a = 1, v = 0, |k| = 1: I - 2kk^T is orthogonal, so |S_t|_F = |S0|_F."""
    d = rand_inputs(1, 50, 2, 8, 6, 11)
    d["beta"].fill_(2.0)
    d["g"].zero_()
    d["v"].zero_()
    d["k"] = d["k"] / d["k"].norm(dim=-1, keepdim=True)
    _, sf = run(orc, d)
    s0 = d["s0"].numpy()
    np.testing.assert_allclose(np.linalg.norm(sf, axis=(2, 3)), np.linalg.norm(s0, axis=(2, 3)),
                               rtol=1e-13)


# --- independent evaluation ---------------------------------------------------------------

@pytest.mark.parametrize("seed,B,T,H,dk,dv,s0", [
    (20, 1, 6, 2, 4, 4, True), (21, 2, 8, 1, 3, 4, False), (22, 1, 7, 3, 4, 2, True),
    (23, 1, 1, 1, 4, 4, True), (24, 1, 0, 2, 3, 3, True)])
def test_p9_brute_force_product_form(orc, seed, B, T, H, dk, dv, s0):
    d = rand_inputs(B, T, H, dk, dv, seed, s0=s0)
    o, sf = run(orc, d)
    ob, sb = orc.brute_force(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sf, sb if d["s0"] is not None or T else np.zeros_like(sf),
                               rtol=0, atol=1e-13)


def test_p9_brute_force_literal_gates_and_large_beta(orc):
    d = rand_inputs(1, 8, 2, 4, 3, 25)
    d["g"] = -torch.nn.functional.softplus(torch.randn(d["g"].shape, dtype=torch.float64) + 3)
    d["beta"] = d["beta"] * 2.0
    o, sf = run(orc, d)
    ob, sb = orc.brute_force(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sf, sb, rtol=0, atol=1e-13)


# --- invariants -----------------------------------------------------------------------------

def test_p6_chaining_is_bitwise(orc):
    """T tokens in one call equal two calls chained through the carried state."""
    d = rand_inputs(2, 37, 3, 8, 8, 6)
    o, sf = run(orc, d)
    for T1 in (1, 16, 23):
        first = {k: x[:, :T1] for k, x in d.items() if k != "s0"}
        first["s0"] = d["s0"]
        o1, s1 = run(orc, first)
        second = {k: x[:, T1:] for k, x in d.items() if k != "s0"}
        second["s0"] = s1
        o2, s2 = run(orc, second)
        assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
        assert np.array_equal(s2, sf)


def test_decode_step_equals_prefill_token_by_token(orc):
    d = rand_inputs(3, 5, 2, 8, 4, 7)
    o, sf = run(orc, d)
    state = d["s0"].numpy().copy()
    for t in range(5):
        ot = orc.decode_step(*(d[x][:, t] for x in ("q", "k", "v", "g", "beta")), state)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(state, sf)


def test_p7_linear_in_state_and_values(orc):
    """For fixed (q, k, g, b) the map (S0, V) -> (O, S_T) is linear."""
    d1 = rand_inputs(1, 30, 2, 8, 6, 8)
    d2 = rand_inputs(1, 30, 2, 8, 6, 9)
    for key in ("q", "k", "g", "beta"):
        d2[key] = d1[key]
    al, be = 0.7, -1.3
    d3 = dict(d1)
    d3["v"] = al * d1["v"] + be * d2["v"]
    d3["s0"] = al * d1["s0"] + be * d2["s0"]
    (o1, s1), (o2, s2), (o3, s3) = run(orc, d1), run(orc, d2), run(orc, d3)
    np.testing.assert_allclose(o3, al * o1 + be * o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(s3, al * s1 + be * s2, rtol=0, atol=1e-13)


def test_p8_value_rows_evolve_independently(orc):
    """Permuting the value dims of V and S0 permutes O and S_T the same way; row subsets agree."""
    d = rand_inputs(2, 25, 2, 6, 7, 10)
    o, sf = run(orc, d)
    perm = np.random.default_rng(0).permutation(7)
    dp = dict(d)
    dp["v"] = d["v"][..., perm]
    dp["s0"] = d["s0"][..., perm]
    op, sp = run(orc, dp)
    assert np.array_equal(op, o[..., perm])
    assert np.array_equal(sp, sf[..., perm])
    rows = [5, 1, 3]
    orr, srr = run(orc, d, rows=rows)
    assert np.array_equal(orr[..., rows], o[..., rows])
    assert np.array_equal(srr[..., rows], sf[..., rows])
    assert np.isnan(orr[..., 0]).all()


def test_p10_contraction_bound(orc):
    """|k| = 1, b in [0,1], a in (0,1]: |S_t|_2 <= a_t |S_{t-1}|_2 + b_t |v_t|."""
    d = rand_inputs(1, 60, 3, 8, 8, 12)
    state = d["s0"].numpy().copy()
    for t in range(60):
        prev = np.linalg.norm(state, ord=2, axis=(2, 3))
        orc.decode_step(*(d[x][:, t] for x in ("q", "k", "v", "g", "beta")), state)
        cur = np.linalg.norm(state, ord=2, axis=(2, 3))
        a = np.exp(d["g"][:, t].numpy())
        bound = a * prev + d["beta"][:, t].numpy() * np.linalg.norm(d["v"][:, t].numpy(), axis=-1)
        assert (cur <= bound * (1 + 1e-12)).all()


def test_state_size_is_independent_of_length(orc):
    """The recurrent state is fixed-size: its shape does not depend on T."""
    for T in (1, 10, 100):
        _, sf = run(orc, rand_inputs(1, T, 2, 4, 3, 13))
        assert sf.shape == (1, 2, 4, 3)


def test_storage_types_widen_exactly(orc):
    """bf16 and fp32 storage give the same result as their exact fp64 widening."""
    d = gi.prefill_inputs(1, 12, 2, 8, 8, wid=901, qkv_dtype=torch.bfloat16, s0=True)
    o_bf, s_bf = run(orc, d)
    d64 = {k: x.to(torch.float64) for k, x in d.items()}
    o64, s64 = run(orc, d64)
    assert np.array_equal(o_bf, o64) and np.array_equal(s_bf, s64)


def test_rejects_bad_arguments(orc):
    d = rand_inputs(1, 4, 1, 4, 4, 14)
    with pytest.raises(ValueError):
        orc.prefill(d["q"], d["k"], d["v"][:, :3], d["g"], d["beta"])
    with pytest.raises(ValueError):
        run(orc, d, rows=[4])


def test_thread_count_does_not_change_results(orc):
    """The oracle's work is split over (batch, head, value row) items that never share a
    result, so one thread and all threads give bit-identical outputs (the CPU baseline times
    both)."""
    d = gi.prefill_inputs(1, 300, 3, 16, 16, wid=902, qkv_dtype=torch.bfloat16, s0=True)
    n = orc.num_threads()
    o_all, s_all = run(orc, d)
    orc.set_num_threads(1)
    try:
        o_one, s_one = run(orc, d)
    finally:
        orc.set_num_threads(n)
    assert orc.num_threads() == n
    assert np.array_equal(o_all, o_one) and np.array_equal(s_all, s_one)
