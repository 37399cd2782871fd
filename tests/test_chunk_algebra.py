"""The chunk form the GPU kernels compute, written out in fp64 NumPy and checked against the
token-by-token oracle (CPU only).

The pages give no chunked algorithm; the kernels use one derived from the rule
S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t / sqrt(d_k) (and, for the
second rule, S_t = a_t S_{t-1} + b_t v_t k_t^T).  For a chunk with start state St = S^T (key-major)
and G_r the cumulative log-gate inside the chunk:

    A = strict_tril(diag(b) (K K^T .* exp(G_r - G_j))),  T = (I + A)^-1   (second rule: T = I)
    W = T diag(b exp G) K,  U = T diag(b) V,  Delta = U - W St           (second rule: Delta = diag(b) V)
    O = scale (diag(exp G) Q St + (Q K^T .* exp(G_r - G_j) .* tril) Delta)
    St' = exp(G_C) St + K^T diag(exp(G_C - G)) Delta

and the state after a run of chunks (a piece) is affine in the state before it,
St_out = M_p St_in + N_p, with N_p the piece run from zeros and M_p the piece run on the identity
with no values.  This file pins that algebra (not the kernels) to the oracle: it is what the chunk
kernel, its piece maps and the chain over pieces implement, so an error in the derivation would
show here before any GPU run.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi

from oracle import GATED_DECAY, GATED_DELTA  # noqa: E402  (rule codes only; no arithmetic)


def chunk_form(q, k, v, g, b, st0, C, rule):
    """One head: q, k [T, dk]; v [T, dv]; g, b [T]; st0 [dk, dv] (key-major). Returns (o, st)."""
    T, dk = k.shape
    scale = 1.0 / np.sqrt(dk)
    st = st0.copy()
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        K, Q, V = k[c0:c0 + C], q[c0:c0 + C], v[c0:c0 + C]
        gg, bb = g[c0:c0 + C], b[c0:c0 + C]
        L = len(gg)
        G = np.cumsum(gg)
        incl = np.tril(np.ones((L, L), dtype=bool))
        # decays exp(G_r - G_j) for j <= r only, masked before the exponential
        decay = np.where(incl, np.exp(np.where(incl, G[:, None] - G[None, :], 0.0)), 0.0)
        if rule == GATED_DELTA:
            A = np.tril(bb[:, None] * (K @ K.T) * decay, -1)
            Tinv = np.linalg.inv(np.eye(L) + A)
            W = Tinv @ ((bb * np.exp(G))[:, None] * K)
            delta = Tinv @ (bb[:, None] * V) - W @ st
        else:
            delta = bb[:, None] * V
        P = (Q @ K.T) * decay
        o[c0:c0 + C] = scale * (np.exp(G)[:, None] * (Q @ st) + P @ delta)
        st = np.exp(G[-1]) * st + K.T @ (np.exp(G[-1] - G)[:, None] * delta)
    return o, st


def inputs(T, dk, dv, seed, gate):
    d = gi.prefill_inputs(1, T, 1, dk, dv, wid=903, call=seed, qkv_dtype=torch.float32, s0=True, gate=gate)
    return {n: (None if x is None else x.to(torch.float64).numpy()) for n, x in d.items()}


def head(d):
    return d["q"][0, :, 0], d["k"][0, :, 0], d["v"][0, :, 0], d["g"][0, :, 0], d["beta"][0, :, 0], d["s0"][0, 0]


def rel(a, ref):
    return float(np.max(np.abs(a - ref)) / np.sqrt(np.mean(ref * ref)))


@pytest.mark.parametrize("rule", [GATED_DELTA, GATED_DECAY])
@pytest.mark.parametrize("gate", ["primary", "literal"])
@pytest.mark.parametrize("C", [1, 16, 32, 64])
@pytest.mark.parametrize("T", [61, 64, 200])
def test_chunk_form_matches_the_token_recurrence(orc, rule, gate, C, T):
    d = inputs(T, 16, 8, seed=C + T, gate=gate)
    ro, rs = orc.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], rule=rule)
    o, st = chunk_form(*head(d), C, rule)
    assert rel(o, ro[0, :, 0]) <= 1e-10, "outputs"
    assert rel(st, rs[0, 0]) <= 1e-10, "final state"


@pytest.mark.parametrize("rule", [GATED_DELTA, GATED_DECAY])
@pytest.mark.parametrize("pieces", [2, 3, 5])
def test_piece_maps_chain_to_the_true_start_states(orc, rule, pieces):
    """Each piece's map (identity columns, no values) and zero-start run, chained over the pieces,
    give every piece's true start state and the final state; each piece rerun from its start
    state gives the true outputs."""
    C, T, dk, dv = 16, 16 * 12 + 5, 16, 8
    d = inputs(T, dk, dv, seed=pieces, gate="primary")
    q, k, v, g, b, s0 = head(d)
    n_chunks = -(-T // C)
    pc = -(-n_chunks // pieces)
    bounds = [min(p * pc * C, T) for p in range(pieces)] + [T]
    st_in, outs = s0.copy(), []
    for p in range(pieces):
        a, e = bounds[p], bounds[p + 1]
        # the oracle's state at the piece boundary: the prefix run token by token
        if a > 0:
            _, rs = orc.prefill(d["q"][:, :a], d["k"][:, :a], d["v"][:, :a], d["g"][:, :a], d["beta"][:, :a],
                                d["s0"], rule=rule)
            assert rel(st_in, rs[0, 0]) <= 1e-10, f"start state of piece {p}"
        o_p, _ = chunk_form(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], st_in, C, rule)
        outs.append(o_p)
        _, n_p = chunk_form(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], np.zeros((dk, dv)), C, rule)
        _, m_p = chunk_form(q[a:e], k[a:e], np.zeros((e - a, dk)), g[a:e], b[a:e], np.eye(dk), C, rule)
        st_in = m_p @ st_in + n_p
    ro, rs = orc.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], rule=rule)
    assert rel(st_in, rs[0, 0]) <= 1e-10, "final state through the chained maps"
    assert rel(np.concatenate(outs), ro[0, :, 0]) <= 1e-10, "outputs of the pieces rerun from their starts"


def test_chunk_form_catches_a_wrong_readout():
    """A planted mistake in the algebra (reading the state before the chunk's writes, i.e.
    dropping the diagonal of P) is far outside the bound: the check has teeth."""
    d = inputs(64, 16, 8, seed=7, gate="primary")
    q, k, v, g, b, s0 = head(d)
    o, _ = chunk_form(q, k, v, g, b, s0, 16, GATED_DELTA)
    o_wrong = o.copy()
    # recompute with the strictly lower P (the output would read S_{t-1})
    scale = 1.0 / np.sqrt(16)
    st = s0.copy()
    for c0 in range(0, 64, 16):
        K, Q, V, gg, bb = k[c0:c0 + 16], q[c0:c0 + 16], v[c0:c0 + 16], g[c0:c0 + 16], b[c0:c0 + 16]
        G = np.cumsum(gg)
        incl = np.tril(np.ones((16, 16), dtype=bool))
        decay = np.where(incl, np.exp(np.where(incl, G[:, None] - G[None, :], 0.0)), 0.0)
        A = np.tril(bb[:, None] * (K @ K.T) * decay, -1)
        Tinv = np.linalg.inv(np.eye(16) + A)
        W = Tinv @ ((bb * np.exp(G))[:, None] * K)
        delta = Tinv @ (bb[:, None] * V) - W @ st
        P = np.tril((Q @ K.T) * decay, -1)
        o_wrong[c0:c0 + 16] = scale * (np.exp(G)[:, None] * (Q @ st) + P @ delta)
        st = np.exp(G[-1]) * st + K.T @ (np.exp(G[-1] - G)[:, None] * delta)
    assert rel(o_wrong, o) > 1e-3


def _piece_map(k, g, b):
    """M_p by the oracle: one head's run on the identity with no values (q and v zero), key-major,
    so that St_out = M_p St_in for a value-free piece."""
    import oracle
    T, dk = k.shape
    z = np.zeros((1, T, 1, dk))
    _, sf = oracle.prefill(z, k[None, :, None, :], z, g[None, :, None], b[None, :, None], np.eye(dk)[None, None])
    return sf[0, 0]


def test_piece_map_drop_bound():
    """The map pass may set a piece map's identity columns to zero once every element is at most
    2^-32, provided every later token's map a (I - b k k^T) has norm at most 1 (g <= 0 and
    b |k|^2 <= 2).  Then what was dropped is only shrunk by the rest of the piece: the piece's end
    state moves by at most d_k max|M| |S| in Frobenius norm.  Pinned here on the oracle: a hard-
    decaying chunk takes the map below 2^-32, a non-expanding chunk after it keeps the dropped
    part within that bound, and a chunk with b |k|^2 = 4 (eigenvalue -3 along k) breaks it, which
    is why such a chunk turns the drops off (and recomputes a map that already dropped)."""
    rng = np.random.default_rng(11)
    dk = dv = 16

    def keys(n, norm2):
        k = rng.standard_normal((n, dk))
        return k / np.linalg.norm(k, axis=1, keepdims=True) * np.sqrt(norm2)

    k1, g1, b1 = keys(32, 1.0), np.full(32, -1.1), rng.uniform(0.2, 1.0, 32)
    m1 = _piece_map(k1, g1, b1)
    tiny = np.max(np.abs(m1))
    assert 0 < tiny <= 2.0 ** -32
    s = rng.standard_normal((dk, dv))
    bound = dk * tiny * np.linalg.norm(s)

    # a chunk that cannot expand the map: the dropped part stays within the bound
    k2, g2, b2 = keys(32, 1.0), np.full(32, -0.03), rng.uniform(0.2, 1.0, 32)
    m2 = _piece_map(k2, g2, b2)
    m = _piece_map(np.concatenate([k1, k2]), np.concatenate([g1, g2]), np.concatenate([b1, b2]))
    assert np.allclose(m, m2 @ m1, rtol=1e-9, atol=1e-12 * tiny)  # maps compose by products
    assert np.linalg.norm(m2, 2) <= 1 + 1e-12
    assert np.linalg.norm(m @ s) <= bound

    # a chunk that can (b = 1, |k|^2 = 4, no decay): the same drop would move the state past it
    k3, g3, b3 = keys(32, 4.0), np.zeros(32), np.ones(32)
    me = _piece_map(np.concatenate([k1, k3]), np.concatenate([g1, g3]), np.concatenate([b1, b3]))
    assert np.linalg.norm(me @ s) > 10 * bound
