"""Closed product form of the gated delta rule, by brute force (tiny inputs only).

TEST INFRASTRUCTURE ONLY.  A second, independent evaluation of the recurrence
used to pin the token-by-token C oracle.  Unrolling

    S_t = S_{t-1} M_t + b_t v_t k_t^T,   M_t = a_t (I - b_t k_t k_t^T),  a_t = exp(g_t)

gives, for every prefix length t,

    S_t = S_0 M_1 M_2 ... M_t + sum_{j<=t} b_j v_j k_j^T M_{j+1} ... M_t
    o_t = S_t q_t / sqrt(d_k)

Each S_t is rebuilt from scratch from explicit d_k x d_k matrix products (no
state is carried from one t to the next), so this shares neither algorithm nor
operation order with the recurrence.  Cost is O(T^3 d^3): keep T and d small.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().cpu().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def brute_force(q, k, v, g, beta, s0=None):
    """q,k [B,T,H,dk]; v [B,T,H,dv]; g,beta [B,T,H]; s0 [B,H,dk,dv] key-major or None.

    Returns (o [B,T,H,dv], s_final [B,H,dk,dv]) in fp64.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    s0 = np.zeros((B, H, dk, dv)) if s0 is None else _f64(s0)
    o = np.zeros((B, T, H, dv))
    sf = np.zeros((B, H, dk, dv))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(H):
            S0 = s0[b, h].T  # math orientation: [dv, dk]
            M = [np.exp(g[b, t, h]) * (eye - beta[b, t, h] * np.outer(k[b, t, h], k[b, t, h]))
                 for t in range(T)]

            def prod(i, j):
                """M_i M_{i+1} ... M_{j-1} (identity when i >= j)."""
                P = eye.copy()
                for m in range(i, j):
                    P = P @ M[m]
                return P

            S = S0
            for t in range(1, T + 1):
                S = S0 @ prod(0, t)
                for j in range(t):
                    S = S + beta[b, j, h] * np.outer(v[b, j, h], k[b, j, h]) @ prod(j + 1, t)
                o[b, t - 1, h] = S @ q[b, t - 1, h] / np.sqrt(dk)
            sf[b, h] = S.T
    return o, sf


def closed_form_decay(q, k, v, g, beta, s0=None):
    """The gated-decay rule S_t = a_t S_{t-1} + b_t v_t k_t^T written out as sums.

    Unrolled, S_t = exp(G_t) S_0 + sum_{j<=t} exp(G_t - G_j) b_j v_j k_j^T with
    G_t = g_1 + ... + g_t, and o_t = S_t q_t / sqrt(d_k).  Every S_t is summed
    from scratch (no carried state).  Same argument conventions as brute_force.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    s0 = np.zeros((B, H, dk, dv)) if s0 is None else _f64(s0)
    o = np.zeros((B, T, H, dv))
    sf = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            G = np.cumsum(g[b, :, h])
            S = s0[b, h].T
            for t in range(T):
                St = np.exp(G[t]) * s0[b, h].T
                for j in range(t + 1):
                    St = St + np.exp(G[t] - G[j]) * beta[b, j, h] * np.outer(v[b, j, h], k[b, j, h])
                o[b, t, h] = St @ q[b, t, h] / np.sqrt(dk)
                S = St
            sf[b, h] = S.T
    return o, sf
