"""fp64 reference of the input preparation ahead of the GDN mixer (TEST INFRASTRUCTURE ONLY).

The pages name the pieces only in passing: when a GDN block replaces an attention layer its
Q/K/V/O projections are copied over while the gates, the decay and a short convolution start
from random values (ftxj.github.io digest of arXiv 2604.24715, Method).  Reading taken (the usual
GDN input path): per token t, head h and channel c

    c_t   = sum_{i=0..3} w[c, i] * x_{t-3+i}[c]        causal depthwise convolution, width 4
                                                       (x_{-3..-1} from a carried state, else 0)
    y_t   = c_t * sigmoid(c_t)                         SiLU
    q_t   = y_t / sqrt(|y_t|^2 + 1e-6)                 over the d_k channels of (t, h); same for k
    v_t   = y_t                                        (value channels: convolution and SiLU only)
    g_t   = -A_h * softplus(a_t + bias_h)              log-gate from a raw logit; A_h > 0 is the
                                                       head's decay rate (1 if absent), bias_h 0 if absent
    b_t   = sigmoid(b_raw_t)                           write strength

Everything is evaluated in fp64 from the stored inputs widened exactly; plain loops over the
definition, no fusion.  Layouts: x [B,T,H,d]; w [H*d, 4] (tap 3 is the current token); a, b_raw
[B,T,H]; conv state [B, H*d, 3] (oldest first).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().cpu().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def short_conv(x, w, state=None):
    """Causal depthwise width-4 convolution. x [B,T,H,d]; w [H*d, 4]; state [B, H*d, 3] or None.
    Returns (c [B,T,H,d], new_state [B, H*d, 3] = the last three inputs, oldest first)."""
    x, w = _f64(x), _f64(w)
    B, T, H, d = x.shape
    flat = x.reshape(B, T, H * d)
    past = np.zeros((B, 3, H * d)) if state is None else np.transpose(_f64(state), (0, 2, 1))
    full = np.concatenate([past, flat], axis=1)  # [B, T + 3, H*d]: full[:, t + 3] = x_t
    c = np.zeros_like(flat)
    for t in range(T):
        for i in range(4):
            c[:, t] += w[:, i] * full[:, t + i]
    new_state = np.transpose(full[:, T:T + 3], (0, 2, 1)).copy()
    return c.reshape(B, T, H, d), new_state


def silu(c):
    return c / (1.0 + np.exp(-c))


def l2norm(y):
    return y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) + EPS)


def prepare(xq, xk, xv, wq, wk, wv, a_raw, b_raw, conv_state=None, A=None, dt_bias=None):
    """Returns dict q, k, v, g, beta (fp64) and conv_state [B, H*(2 d_k + d_v), 3]; conv_state
    channels are ordered q channels, then k, then v (each h-major, as the projections).
    A, dt_bias: per-head [H] or None."""
    B, T, H, dk = _f64(xq).shape
    dv = _f64(xv).shape[-1]
    sq = sk = sv = None
    if conv_state is not None:
        cs = _f64(conv_state)
        sq, sk, sv = cs[:, :H * dk], cs[:, H * dk:2 * H * dk], cs[:, 2 * H * dk:]
    cq, nq = short_conv(xq, wq, sq)
    ck, nk = short_conv(xk, wk, sk)
    cv, nv = short_conv(xv, wv, sv)
    a, br = _f64(a_raw), _f64(b_raw)
    rate = np.ones(H) if A is None else _f64(A)
    bias = np.zeros(H) if dt_bias is None else _f64(dt_bias)
    z = a + bias
    softplus = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))  # log(1 + e^z) without overflow
    return {
        "q": l2norm(silu(cq)), "k": l2norm(silu(ck)), "v": silu(cv),
        "g": -rate * softplus, "beta": 1.0 / (1.0 + np.exp(-br)),
        "conv_state": np.concatenate([nq, nk, nv], axis=1),
    }
