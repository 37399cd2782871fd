"""Seeded synthetic inputs for the GDN token mixer.

Shared by the tests, the smoke check and the benchmark.  This module holds no
arithmetic of the method itself: it only draws random tensors with the shapes,
dtypes and value distributions of the workloads below, so that the GPU path
and the CPU oracle are fed the very same stored values.

Workloads (layer shapes of the pages' base models; context lengths of their
RULER evaluations and of their 2M-token serving runs -- ftxj.github.io digest
of arXiv 2604.24715, Experiments, Results and Figure 5):

* ``tiny``    B=1, H=2,  T=64,     d_k=d_v=16,  fp32 everything, chunk 16, zero start state
* ``1b_8k``   B=4, H=32, T=8192,   d=64,  bf16 q/k/v, chunk 64, zero start state
* ``1b_64k``  B=1, H=32, T=65536,  d=64,  bf16 q/k/v, chunk 64, start state 0.1*N(0,1)
* ``3b_2m``   B=1, H=24, T=65536 per call x 32 chained calls, d=128, bf16, chunk 64
* ``decode``  N=256 sequences, H=32, d=64, 16 single-token steps, state 0.1*N(0,1)

Value recipe (all fp32 before any bf16 rounding, which is round-to-nearest-even):
q, k ~ N(0,1) then L2-normalised per (token, head); v ~ N(0,1);
beta = sigmoid(N(0,1)); log-gate g = -softplus(N(0,1) - shift) with shift 3
(median decay a = exp(g) = sigmoid(3) = 0.953) or 4 for the 3B shape
(median a = 0.982).  ``gate="literal"`` uses -softplus(N(0,1) + shift) instead
(median a = 0.047), kept as a numerical stress case.  Start states are
0.1*N(0,1).

Seeds: every tensor has its own torch generator seeded from
(workload id, call or step index, tensor id), so tensors of a long chained
workload can be drawn one call at a time.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "beta": 3, "g": 4, "s0": 5, "xq": 6, "xk": 7, "xv": 8, "conv_w": 9,
              "a_raw": 10, "b_raw": 11, "rate": 12, "dt": 13, "conv_state": 14}


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    qkv_dtype: torch.dtype
    gate_shift: float
    s0: bool
    calls: int = 1  # chained prefill calls (3b_2m) or decode steps (decode)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 2, 64, 16, 16, 16, torch.float32, 3.0, False),
    "1b_8k": Workload("1b_8k", 2, 4, 32, 8192, 64, 64, 64, torch.bfloat16, 3.0, False),
    "1b_64k": Workload("1b_64k", 3, 1, 32, 65536, 64, 64, 64, torch.bfloat16, 3.0, True),
    "3b_2m": Workload("3b_2m", 4, 1, 24, 65536, 128, 128, 64, torch.bfloat16, 4.0, False, calls=32),
    "decode": Workload("decode", 5, 256, 32, 1, 64, 64, 1, torch.bfloat16, 3.0, True, calls=16),
}


def seed_of(wid: int, call: int, tensor: str) -> int:
    return (wid << 40) | (call << 8) | TENSOR_IDS[tensor]


def _normal(shape, seed, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def draw_qk(shape, seed, dtype, device):
    x = _normal(shape, seed, device)
    x = x / x.norm(dim=-1, keepdim=True)
    return x.to(dtype)


def draw_v(shape, seed, dtype, device):
    return _normal(shape, seed, device).to(dtype)


def draw_beta(shape, seed, device):
    return torch.sigmoid(_normal(shape, seed, device))


def draw_gate(shape, seed, shift, device, gate="primary"):
    x = _normal(shape, seed, device)
    if gate == "primary":
        return -torch.nn.functional.softplus(x - shift)
    if gate == "literal":
        return -torch.nn.functional.softplus(x + shift)
    raise ValueError(f"unknown gate reading {gate!r}")


def draw_state(shape, seed, device):
    return 0.1 * _normal(shape, seed, device)


def prefill_inputs(B, T, H, dk, dv, *, wid=0, call=0, qkv_dtype=torch.bfloat16, gate_shift=3.0,
                   gate="primary", s0=False, device="cpu"):
    """Draw one prefill call's inputs: dict with q, k, v, g, beta, s0 (or None)."""
    d = {
        "q": draw_qk((B, T, H, dk), seed_of(wid, call, "q"), qkv_dtype, device),
        "k": draw_qk((B, T, H, dk), seed_of(wid, call, "k"), qkv_dtype, device),
        "v": draw_v((B, T, H, dv), seed_of(wid, call, "v"), qkv_dtype, device),
        "beta": draw_beta((B, T, H), seed_of(wid, call, "beta"), device),
        "g": draw_gate((B, T, H), seed_of(wid, call, "g"), gate_shift, device, gate),
        "s0": draw_state((B, H, dk, dv), seed_of(wid, call, "s0"), device) if s0 else None,
    }
    return d


def workload_inputs(name, call=0, *, gate="primary", device="cpu", T=None, B=None, H=None):
    """Inputs of one call (prefill workloads) of a named workload.

    T, B, H may be overridden to draw a reduced sample of the same recipe.
    The start state of the 3B chain is drawn only for call 0 when requested
    (the chain starts from zeros).
    """
    w = WORKLOADS[name]
    return prefill_inputs(B or w.B, T or w.T, H or w.H, w.dk, w.dv, wid=w.wid, call=call,
                          qkv_dtype=w.qkv_dtype, gate_shift=w.gate_shift, gate=gate,
                          s0=w.s0, device=device)


def decode_inputs(N, H, dk, dv, step, *, wid=5, qkv_dtype=torch.bfloat16, gate_shift=3.0,
                  gate="primary", device="cpu"):
    """One decode step's inputs: q, k [N,H,dk], v [N,H,dv], g, beta [N,H]."""
    return {
        "q": draw_qk((N, H, dk), seed_of(wid, step, "q"), qkv_dtype, device),
        "k": draw_qk((N, H, dk), seed_of(wid, step, "k"), qkv_dtype, device),
        "v": draw_v((N, H, dv), seed_of(wid, step, "v"), qkv_dtype, device),
        "beta": draw_beta((N, H), seed_of(wid, step, "beta"), device),
        "g": draw_gate((N, H), seed_of(wid, step, "g"), gate_shift, device, gate),
    }


def decode_state(N, H, dk, dv, *, wid=5, device="cpu"):
    return draw_state((N, H, dk, dv), seed_of(wid, 0, "s0"), device)


def _uniform(shape, seed, lo, hi, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return lo + (hi - lo) * torch.rand(shape, generator=gen, device=device, dtype=torch.float32)


def prep_inputs(B, T, H, dk, dv, *, wid=0, call=0, x_dtype=torch.bfloat16, state=True, rate=True,
                device="cpu"):
    """Raw inputs of the preparation ahead of the mixer (the projections' outputs and the block's
    own parameters), as a randomly initialised converted block would hold them:

    xq, xk [B,T,H,dk], xv [B,T,H,dv] ~ N(0,1) in x_dtype; conv_weight [H*(2dk+dv), 4] ~ U(-1/2, 1/2)
    (fan-in 4); a_raw, b_raw [B,T,H] ~ N(0,1); decay_rate [H] ~ U(1, 16); gate_bias [H] = the inverse
    softplus of dt ~ exp(U(log 1e-3, log 1e-1)); conv_state [B, H*(2dk+dv), 3] ~ N(0,1) rounded
    through x_dtype (it holds earlier raw inputs).  ``state=False`` / ``rate=False`` give None for
    the state / for decay_rate and gate_bias."""
    C = H * (2 * dk + dv)
    d = {
        "xq": _normal((B, T, H, dk), seed_of(wid, call, "xq"), device).to(x_dtype),
        "xk": _normal((B, T, H, dk), seed_of(wid, call, "xk"), device).to(x_dtype),
        "xv": _normal((B, T, H, dv), seed_of(wid, call, "xv"), device).to(x_dtype),
        "conv_weight": _uniform((C, 4), seed_of(wid, 0, "conv_w"), -0.5, 0.5, device),
        "a_raw": _normal((B, T, H), seed_of(wid, call, "a_raw"), device),
        "b_raw": _normal((B, T, H), seed_of(wid, call, "b_raw"), device),
        "decay_rate": None, "gate_bias": None, "conv_state": None,
    }
    if rate:
        d["decay_rate"] = _uniform((H,), seed_of(wid, 0, "rate"), 1.0, 16.0, device)
        dt = torch.exp(_uniform((H,), seed_of(wid, 0, "dt"), -6.907755, -2.302585, device))
        d["gate_bias"] = dt + torch.log(-torch.expm1(-dt))
    if state:
        d["conv_state"] = _normal((B, C, 3), seed_of(wid, call, "conv_state"), device).to(x_dtype).float()
    return d
