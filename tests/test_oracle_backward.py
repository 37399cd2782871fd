"""Pins of the oracle's gradients (CPU only).

The backward oracle (the token-by-token adjoint in gdn_oracle.c) is checked against things it
shares no code with:
  * central finite differences of the forward oracle on L = sum <d_o, o> + <ds_final, S_T>, every
    input element, both rules, across a checkpoint boundary of the state recomputation;
  * reverse-mode automatic differentiation (torch, fp64) of the matrix recurrence written out here
    from the rule's definition;
  * linearity of every gradient in (d_o, ds_final), and T = 0 (ds0 = ds_final).
Plausible mistakes planted in copies of the C source (dropped symmetric term, erase sign, missing
gate factor, undecayed adjoint, readout gradient on the wrong state) must each fail a pin.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle.build import SRC

NAMES = ("q", "k", "v", "g", "beta", "s0")
GRADS = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "s0": "ds0"}


def inputs(seed, B, T, H, dk, dv):
    rng = np.random.default_rng(seed)
    x = {
        "q": rng.normal(size=(B, T, H, dk)) / np.sqrt(dk),
        "k": rng.normal(size=(B, T, H, dk)) / np.sqrt(dk),
        "v": rng.normal(size=(B, T, H, dv)),
        "g": -np.abs(rng.normal(size=(B, T, H))) * 0.3,
        "beta": rng.uniform(0.1, 1.0, size=(B, T, H)),
        "s0": rng.normal(size=(B, H, dk, dv)) * 0.3,
    }
    d_o = rng.normal(size=(B, T, H, dv))
    ds = rng.normal(size=(B, H, dk, dv))
    return x, d_o, ds


def loss(orc, x, d_o, ds, rule):
    o, sf = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], rule=rule)
    return float(np.sum(o * d_o) + np.sum(sf * ds))


def fd_check(orc, rule, seed, B, T, H, dk, dv, names=NAMES, tol=1e-7):
    x, d_o, ds = inputs(seed, B, T, H, dk, dv)
    got = orc.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o, ds, rule=rule)
    eps = 1e-6
    for n in names:
        fd = np.zeros_like(x[n])
        for idx in np.ndindex(x[n].shape):
            keep = x[n][idx]
            x[n][idx] = keep + eps
            lp = loss(orc, x, d_o, ds, rule)
            x[n][idx] = keep - eps
            lm = loss(orc, x, d_o, ds, rule)
            x[n][idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - got[GRADS[n]])) / max(1.0, np.max(np.abs(fd)))
        assert err < tol, (n, rule, err)


@pytest.mark.parametrize("rule", [oracle.GATED_DELTA, oracle.GATED_DECAY])
def test_gradients_match_finite_differences(rule, orc=None):
    fd_check(orc or oracle.default(), rule, 1, 2, 5, 2, 3, 2)


def test_gradients_across_a_checkpoint_boundary(orc=None):
    # T = 70 > the 64-token checkpoint spacing of the state recomputation
    fd_check(orc or oracle.default(), oracle.GATED_DELTA, 2, 1, 70, 1, 2, 2, names=("k", "g", "beta", "s0"))


def torch_grads(x, d_o, ds, rule):
    """Reverse-mode AD of S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T (or without the
    erase term), o_t = S_t q_t / sqrt(d_k), with S [d_v, d_k]; states key-major outside."""
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in x.items()}
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    eye = torch.eye(dk, dtype=torch.float64)
    S = t["s0"].transpose(-1, -2)  # [B, H, dv, dk]
    outs = []
    for i in range(T):
        q, k, v = t["q"][:, i], t["k"][:, i], t["v"][:, i]
        a = torch.exp(t["g"][:, i])[..., None, None]
        b = t["beta"][:, i][..., None, None]
        kk = k[..., :, None] * k[..., None, :]
        M = a * (eye - b * kk) if rule == oracle.GATED_DELTA else a * eye
        S = S @ M + b * (v[..., :, None] * k[..., None, :])
        outs.append((S @ q[..., :, None])[..., 0] / np.sqrt(dk))
    o = torch.stack(outs, dim=1)
    L = (o * torch.tensor(d_o)).sum() + (S.transpose(-1, -2) * torch.tensor(ds)).sum()
    L.backward()
    return {GRADS[n]: t[n].grad.numpy() for n in NAMES}


@pytest.mark.parametrize("rule", [oracle.GATED_DELTA, oracle.GATED_DECAY])
def test_gradients_match_autograd_of_the_recurrence(rule):
    x, d_o, ds = inputs(3, 2, 40, 2, 8, 6)
    got = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o, ds, rule=rule)
    ref = torch_grads(x, d_o, ds, rule)
    for n, r in ref.items():
        np.testing.assert_allclose(got[n], r, rtol=1e-10, atol=1e-12 * max(1.0, np.max(np.abs(r))), err_msg=n)


def test_gradients_are_linear_in_the_upstream_gradients():
    x, d1, s1 = inputs(4, 1, 9, 2, 4, 4)
    _, d2, s2 = inputs(5, 1, 9, 2, 4, 4)
    f = lambda d, s: oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d, s)
    a, b, c = f(d1, s1), f(d2, s2), f(d1 + 2 * d2, s1 + 2 * s2)
    for n in a:
        np.testing.assert_allclose(c[n], a[n] + 2 * b[n], rtol=1e-12, atol=1e-12, err_msg=n)


def test_zero_tokens_pass_the_state_gradient_through():
    x, d_o, ds = inputs(6, 2, 0, 3, 4, 4)
    got = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o, ds)
    assert np.array_equal(got["ds0"], ds)
    got = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o, None)
    assert np.array_equal(got["ds0"], np.zeros_like(ds))


# (name, original text, planted mistake)
MUTANTS = [
    ("bwd_drop_symmetric_term", "(dMk[j] + dMtk[j])", "(dMk[j])"),
    ("bwd_erase_sign", "da -= bt * kdk;", "da += bt * kdk;"),
    ("bwd_gate_factor", "dg[bth] = a * da;", "dg[bth] = da;"),
    ("bwd_adjoint_not_decayed", "D[i * dk + j] = a * (D[i * dk + j] -", "D[i * dk + j] = (D[i * dk + j] -"),
    ("bwd_readout_previous_state", "acc += St[i * dk + j] * dot[i];", "acc += Sp[i * dk + j] * dot[i];"),
    ("bwd_beta_erase_part", "db -= a * kdk;", "db -= kdk;"),
    ("bwd_write_grad_unscaled", "dv_out[bth * dv + i] = bt * Dk[i];", "dv_out[bth * dv + i] = Dk[i];"),
]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_backward_mistake(tmp_path, name, orig, bad):
    with open(SRC) as f:
        src = f.read()
    assert src.count(orig) == 1, f"mutation site for {name} not unique"
    csrc, lib = tmp_path / f"{name}.c", tmp_path / f"lib{name}.so"
    csrc.write_text(src.replace(orig, bad))
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(lib), str(csrc), "-lm"],
                   check=True)
    mutant = oracle.Oracle(str(lib))
    failed = []
    for rule in (oracle.GATED_DELTA, oracle.GATED_DECAY):
        try:
            fd_check(mutant, rule, 1, 1, 4, 2, 3, 2)
        except AssertionError:
            failed.append(rule)
    assert failed, f"no pin detects the planted mistake {name!r}"
