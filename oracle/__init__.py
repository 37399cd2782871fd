"""fp64 CPU oracle of the Gated DeltaNet token mixer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the GPU library.

Two independent evaluations of the gated delta rule are provided:

* ``prefill`` / ``decode_step`` -- the token-by-token recurrence in C
  (``gdn_oracle.c``), fp64, OpenMP over (batch, head, value row).
* ``brute_force`` (``oracle.brute``) -- the closed product form of the same
  recurrence, by explicit matrix products in NumPy; for tiny inputs only.

The rule (the pages give it in words only: the kwkr.cn digest of
HyLo-Llama-8MLA8GDN-8K-SFT, architecture section, calls the GDN layer a gated
delta-rule linear attention with a fixed-size recurrent state; the we0.ai
Priming article, SSM comparison, says it erases or rewrites the value held
under a key):

    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   a_t = exp(g_t)
    o_t = S_t q_t / sqrt(d_k)

A second rule, ``rule=GATED_DECAY``, drops the erase term: S_t = a_t S_{t-1} + b_t v_t k_t^T
(the uniform decay the Priming article attributes to Mamba-2).  ``closed_form_decay``
(``oracle.brute``) evaluates it as explicit decayed sums, independently of the recurrence.

``backward`` gives the gradients of L = sum_t <d_o_t, o_t> + <dS_T, S_T> by the token-by-token
adjoint of the recurrence (C, fp64).

States are stored key-major, ``[..., d_k, d_v]`` (element (j, i) = S[i][j]).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .brute import brute_force, closed_form_decay
from . import prep
from .build import LIB, build

F64, F32, BF16 = 0, 1, 2
GATED_DELTA, GATED_DECAY = 0, 1  # the rules the oracle evaluates


def _as_array(x):
    """Return (contiguous numpy array of the stored values or bits, dtype code)."""
    if x is None:
        return None, F64
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                x = x.cpu()
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            x = x.numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:  # raw bf16 bits
        return x, BF16
    raise TypeError(f"oracle: unsupported dtype {x.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes front end of one build of ``gdn_oracle.c`` (the default build, or
    a test-only variant compiled elsewhere)."""

    def __init__(self, path: str = LIB):
        lib = ctypes.CDLL(path)
        vp, dp, lg, i32 = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_long, ctypes.c_int
        lib.gdn_oracle_prefill_rule.argtypes = [i32, vp, vp, vp, i32, vp, vp, i32, vp, i32, dp, dp,
                                                lg, lg, lg, lg, lg, ctypes.POINTER(ctypes.c_int), lg]
        lib.gdn_oracle_prefill_rule.restype = i32
        lib.gdn_oracle_decode_step_rule.argtypes = [i32, vp, vp, vp, i32, vp, vp, i32, dp, dp,
                                                    lg, lg, lg, lg]
        lib.gdn_oracle_decode_step_rule.restype = i32
        lib.gdn_oracle_backward_rule.argtypes = [i32, vp, vp, vp, i32, vp, vp, i32, vp, i32, vp, vp, i32,
                                                 dp, dp, dp, dp, dp, dp, lg, lg, lg, lg, lg]
        lib.gdn_oracle_backward_rule.restype = i32
        lib.gdn_oracle_num_threads.argtypes = []
        lib.gdn_oracle_num_threads.restype = i32
        lib.gdn_oracle_set_num_threads.argtypes = [i32]
        lib.gdn_oracle_set_num_threads.restype = None
        self.lib = lib
        self.brute_force = brute_force
        self.closed_form_decay = closed_form_decay

    def num_threads(self) -> int:
        return int(self.lib.gdn_oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        """Threads of the following calls (timing only; results do not depend on it)."""
        self.lib.gdn_oracle_set_num_threads(int(n))

    def prefill(self, q, k, v, g, beta, s0=None, rows=None, rule=GATED_DELTA):
        """Token-by-token fp64 evaluation of ``rule`` (GATED_DELTA or GATED_DECAY).

        q, k: [B,T,H,d_k]; v: [B,T,H,d_v]; g, beta: [B,T,H]; s0: [B,H,d_k,d_v] or None (zeros).
        rows: optional list of value rows to evaluate (others are left NaN).
        Returns (o [B,T,H,d_v] fp64, s_final [B,H,d_k,d_v] fp64).
        """
        qa, qd = _as_array(q)
        ka, kd = _as_array(k)
        va, vd = _as_array(v)
        if not (qd == kd == vd):
            raise TypeError("oracle: q, k, v must share one storage type")
        ga, gd = _as_array(g)
        ba, bd = _as_array(beta)
        if gd != bd:
            raise TypeError("oracle: g and beta must share one storage type")
        sa, sd = _as_array(s0)
        B, T, H, dk = qa.shape
        dv = va.shape[-1]
        if ka.shape != (B, T, H, dk) or va.shape != (B, T, H, dv):
            raise ValueError("oracle: q/k/v shape mismatch")
        if ga.shape != (B, T, H) or ba.shape != (B, T, H):
            raise ValueError("oracle: g/beta shape mismatch")
        if sa is not None and sa.shape != (B, H, dk, dv):
            raise ValueError("oracle: s0 shape mismatch")
        o = np.full((B, T, H, dv), np.nan)
        sf = np.full((B, H, dk, dv), np.nan)
        if rows is not None:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
            rp, nr = rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), len(rows_arr)
        else:
            rows_arr, rp, nr = None, None, 0
        dp = ctypes.POINTER(ctypes.c_double)
        rc = self.lib.gdn_oracle_prefill_rule(rule, _ptr(qa), _ptr(ka), _ptr(va), qd, _ptr(ga), _ptr(ba),
                                              gd, _ptr(sa), sd, o.ctypes.data_as(dp),
                                              sf.ctypes.data_as(dp), B, T, H, dk, dv, rp, nr)
        if rc != 0:
            raise ValueError("oracle: gdn_oracle_prefill rejected its arguments")
        return o, sf

    def decode_step(self, q, k, v, g, beta, state, rule=GATED_DELTA):
        """One single-token step of ``rule`` for N sequences.

        q, k: [N,H,d_k]; v: [N,H,d_v]; g, beta: [N,H]; state: [N,H,d_k,d_v] fp64 numpy,
        updated in place.  Returns o [N,H,d_v] fp64.
        """
        qa, qd = _as_array(q)
        ka, _ = _as_array(k)
        va, _ = _as_array(v)
        ga, gd = _as_array(g)
        ba, _ = _as_array(beta)
        if not (isinstance(state, np.ndarray) and state.dtype == np.float64
                and state.flags.c_contiguous):
            raise TypeError("oracle: decode state must be a contiguous fp64 numpy array")
        N, H, dk = qa.shape
        dv = va.shape[-1]
        if state.shape != (N, H, dk, dv):
            raise ValueError("oracle: state shape mismatch")
        o = np.full((N, H, dv), np.nan)
        dp = ctypes.POINTER(ctypes.c_double)
        rc = self.lib.gdn_oracle_decode_step_rule(rule, _ptr(qa), _ptr(ka), _ptr(va), qd, _ptr(ga),
                                                  _ptr(ba), gd, state.ctypes.data_as(dp),
                                                  o.ctypes.data_as(dp), N, H, dk, dv)
        if rc != 0:
            raise ValueError("oracle: gdn_oracle_decode_step rejected its arguments")
        return o


    def backward(self, q, k, v, g, beta, s0, d_o, ds_final=None, rule=GATED_DELTA):
        """Gradients of L = sum_t <d_o_t, o_t> + <ds_final, S_T> for ``rule``, fp64, by the
        token-by-token adjoint of the recurrence (states recomputed from checkpoints).

        Shapes as ``prefill``; d_o [B,T,H,d_v]; ds_final [B,H,d_k,d_v] or None (zero), d_o and
        ds_final in one storage type.  Returns a dict of fp64 arrays dq, dk [B,T,H,d_k],
        dv [B,T,H,d_v], dg, dbeta [B,T,H], ds0 [B,H,d_k,d_v].
        """
        qa, qd = _as_array(q)
        ka, kd = _as_array(k)
        va, vd = _as_array(v)
        if not (qd == kd == vd):
            raise TypeError("oracle: q, k, v must share one storage type")
        ga, gd = _as_array(g)
        ba, bd = _as_array(beta)
        if gd != bd:
            raise TypeError("oracle: g and beta must share one storage type")
        sa, sd = _as_array(s0)
        oa, od = _as_array(d_o)
        fa, fd = _as_array(ds_final)
        if fa is not None and fd != od:
            raise TypeError("oracle: d_o and ds_final must share one storage type")
        B, T, H, dk = qa.shape
        dv = va.shape[-1]
        if oa.shape != (B, T, H, dv) or (fa is not None and fa.shape != (B, H, dk, dv)):
            raise ValueError("oracle: gradient shape mismatch")
        if sa is not None and sa.shape != (B, H, dk, dv):
            raise ValueError("oracle: s0 shape mismatch")
        out = {"dq": np.full((B, T, H, dk), np.nan), "dk": np.full((B, T, H, dk), np.nan),
               "dv": np.full((B, T, H, dv), np.nan), "dg": np.full((B, T, H), np.nan),
               "dbeta": np.full((B, T, H), np.nan), "ds0": np.full((B, H, dk, dv), np.nan)}
        dp = ctypes.POINTER(ctypes.c_double)
        rc = self.lib.gdn_oracle_backward_rule(rule, _ptr(qa), _ptr(ka), _ptr(va), qd, _ptr(ga), _ptr(ba), gd,
                                               _ptr(sa), sd, _ptr(oa), _ptr(fa), od,
                                               *[out[n].ctypes.data_as(dp) for n in ("dq", "dk", "dv", "dg",
                                                                                     "dbeta", "ds0")],
                                               B, T, H, dk, dv)
        if rc != 0:
            raise ValueError("oracle: gdn_oracle_backward rejected its arguments")
        return out


_default = None


def default() -> Oracle:
    """The oracle library the tests use: the default build, or the one GDN_ORACLE_LIB names (a
    sanitizer build of the same source, loaded by the sanitizer test)."""
    global _default
    if _default is None:
        path = os.environ.get("GDN_ORACLE_LIB", "")
        if not path:
            path = LIB
            if not os.path.exists(LIB):
                build()
        _default = Oracle(path)
    return _default


def prefill(*args, **kw):
    return default().prefill(*args, **kw)


def decode_step(*args, **kw):
    return default().decode_step(*args, **kw)


def backward(*args, **kw):
    return default().backward(*args, **kw)


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


__all__ = ["Oracle", "default", "prefill", "decode_step", "backward", "brute_force", "closed_form_decay", "prep",
           "num_threads", "set_num_threads", "build", "GATED_DELTA", "GATED_DECAY"]
