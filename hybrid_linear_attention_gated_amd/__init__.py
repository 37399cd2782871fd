"""Python binding of libgdn, the Gated DeltaNet token mixer for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgdn.so``.  PyTorch supplies device memory and the stream.

Raw C-ABI entry points (same names and arguments as ``include/gdn.h``, with
pointers passed as integers):

    gdn_chunk_prefill, gdn_chunk_prefill_rule, gdn_chunk_prefill_workspace_size, gdn_chunk_prefill_noalloc,
    gdn_chunk_prefill_varlen, gdn_chunk_prefill_varlen_workspace_size, gdn_decode_step,
    gdn_decode_step_rule, gdn_decode_step_slots, gdn_prepare, gdn_prepare_decode_step,
    gdn_chunk_backward, gdn_chunk_backward_workspace_size, gdn_status_string, gdn_version

Tensor helpers that allocate outputs with torch and call the above on the
current stream:

    chunk_prefill(q, k, v, g, beta, initial_state=None, chunk=64) -> (o, final_state)
    decode_step(q, k, v, g, beta, state) -> o        (state updated in place)
    decode_step_slots / chunk_prefill_varlen          (states in a pool, packed sequences)
    prepare(xq, xk, xv, conv_weight, a_raw, b_raw) -> (q, k, v, g, beta)
    prepare_decode_step(xq, xk, xv, conv_weight, a_raw, b_raw, conv_state, state) -> o
    prepare_chunk_prefill(xq, xk, xv, conv_weight, a_raw, b_raw, initial_state) -> (o, final_state)
    chunk_backward(q, k, v, g, beta, d_o, ...) -> (dq, dk, dv, dg, dbeta, d_initial_state)

The rule computed (a gated delta rule; the pages describe the GDN layer in
words only -- kwkr.cn digest of HyLo-Llama-8MLA8GDN-8K-SFT, architecture
section; we0.ai Priming article, SSM comparison):

    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  a_t = exp(g_t)
    o_t = S_t q_t / sqrt(d_k)
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_RULE_GATED_DELTA, GDN_RULE_GATED_DECAY = 0, 1
STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
          4: "GDN_ERR_ALIGN", 5: "GDN_ERR_ALIAS", 6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_HIP",
          8: "GDN_ERR_CAPTURE"}
EXPORTS = ("gdn_chunk_prefill", "gdn_chunk_prefill_rule", "gdn_chunk_prefill_workspace_size",
           "gdn_chunk_prefill_noalloc",
           "gdn_chunk_prefill_varlen", "gdn_chunk_prefill_varlen_workspace_size",
           "gdn_decode_step", "gdn_decode_step_rule", "gdn_decode_step_slots", "gdn_prepare",
           "gdn_chunk_backward", "gdn_chunk_backward_workspace_size", "gdn_prepare_varlen",
           "gdn_prepare_varlen_workspace_size", "gdn_prepare_decode_step", "gdn_prepare_chunk_prefill",
           "gdn_prepare_chunk_prefill_workspace_size", "gdn_status_string", "gdn_version")


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gdn_status_string(status)}")


_lib = None


def lib():
    """The loaded libgdn.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libgdn.so is not built ({LIB_PATH}); run "
                               "`python -m hybrid_linear_attention_gated_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.gdn_chunk_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                        i32, vp, sz, vp]
        L.gdn_chunk_prefill.restype = i32
        L.gdn_chunk_prefill_rule.argtypes = [i32] + L.gdn_chunk_prefill.argtypes
        L.gdn_chunk_prefill_rule.restype = i32
        L.gdn_chunk_prefill_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                i32, i32, vp]
        L.gdn_chunk_prefill_noalloc.restype = i32
        L.gdn_chunk_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.gdn_chunk_prefill_workspace_size.restype = sz
        L.gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        L.gdn_decode_step.restype = i32
        L.gdn_decode_step_rule.argtypes = [i32] + L.gdn_decode_step.argtypes
        L.gdn_decode_step_rule.restype = i32
        L.gdn_decode_step_slots.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                            i32, vp]
        L.gdn_decode_step_slots.restype = i32
        L.gdn_chunk_prefill_varlen.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp,
                                               i32, i32, i32, i32, i32, vp, sz, vp]
        L.gdn_chunk_prefill_varlen.restype = i32
        L.gdn_chunk_prefill_varlen_workspace_size.argtypes = [vp, i32, i32, i32, i32, i32, i32]
        L.gdn_chunk_prefill_varlen_workspace_size.restype = sz
        L.gdn_prepare.argtypes = [vp] * 15 + [i32] * 6 + [vp]
        L.gdn_prepare.restype = i32
        L.gdn_prepare_decode_step.argtypes = [i32] + [vp] * 11 + [i32] * 5 + [vp]
        L.gdn_prepare_decode_step.restype = i32
        L.gdn_chunk_backward.argtypes = [i32] + [vp] * 14 + [i32] * 6 + [vp, sz, vp]
        L.gdn_chunk_backward.restype = i32
        L.gdn_chunk_backward_workspace_size.argtypes = [i32] * 6
        L.gdn_chunk_backward_workspace_size.restype = sz
        L.gdn_prepare_varlen.argtypes = [vp] * 9 + [i32, i32, vp, i32, vp, vp] + [vp] * 5 + [i32] * 4 + [vp, sz, vp]
        L.gdn_prepare_varlen.restype = i32
        L.gdn_prepare_varlen_workspace_size.argtypes = [i32]
        L.gdn_prepare_varlen_workspace_size.restype = sz
        L.gdn_prepare_chunk_prefill.argtypes = [i32] + [vp] * 13 + [i32] * 7 + [vp, sz, vp]
        L.gdn_prepare_chunk_prefill.restype = i32
        L.gdn_prepare_chunk_prefill_workspace_size.argtypes = [i32] * 7
        L.gdn_prepare_chunk_prefill_workspace_size.restype = sz
        L.gdn_status_string.argtypes = [i32]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_version.argtypes = []
        L.gdn_version.restype = i32
        _lib = L
    return _lib


# ---- raw C-ABI entry points ----------------------------------------------------------

def gdn_chunk_prefill(q, k, v, g, beta, initial_state, o, final_state, B, T, H, d_k, d_v, chunk,
                      qkv_dtype, workspace, workspace_bytes, stream) -> int:
    return lib().gdn_chunk_prefill(q, k, v, g, beta, initial_state, o, final_state, B, T, H, d_k,
                                   d_v, chunk, qkv_dtype, workspace, workspace_bytes, stream)


def gdn_chunk_prefill_rule(rule, q, k, v, g, beta, initial_state, o, final_state, B, T, H, d_k, d_v,
                           chunk, qkv_dtype, workspace, workspace_bytes, stream) -> int:
    return lib().gdn_chunk_prefill_rule(rule, q, k, v, g, beta, initial_state, o, final_state, B, T, H,
                                        d_k, d_v, chunk, qkv_dtype, workspace, workspace_bytes, stream)


def gdn_chunk_prefill_noalloc(rule, q, k, v, g, beta, initial_state, o, final_state, B, T, H, d_k, d_v, chunk,
                              qkv_dtype, stream) -> int:
    return lib().gdn_chunk_prefill_noalloc(rule, q, k, v, g, beta, initial_state, o, final_state, B, T, H, d_k,
                                           d_v, chunk, qkv_dtype, stream)


def gdn_chunk_prefill_workspace_size(B, T, H, d_k, d_v, chunk, qkv_dtype) -> int:
    return lib().gdn_chunk_prefill_workspace_size(B, T, H, d_k, d_v, chunk, qkv_dtype)


def gdn_decode_step(q, k, v, g, beta, state, o, N, H, d_k, d_v, qkv_dtype, stream) -> int:
    return lib().gdn_decode_step(q, k, v, g, beta, state, o, N, H, d_k, d_v, qkv_dtype, stream)


def gdn_decode_step_rule(rule, q, k, v, g, beta, state, o, N, H, d_k, d_v, qkv_dtype, stream) -> int:
    return lib().gdn_decode_step_rule(rule, q, k, v, g, beta, state, o, N, H, d_k, d_v, qkv_dtype,
                                      stream)


def gdn_decode_step_slots(rule, q, k, v, g, beta, state_pool, slots, pool_size, o, N, H, d_k, d_v,
                          qkv_dtype, stream) -> int:
    return lib().gdn_decode_step_slots(rule, q, k, v, g, beta, state_pool, slots, pool_size, o, N, H,
                                       d_k, d_v, qkv_dtype, stream)


def gdn_chunk_prefill_varlen(rule, q, k, v, g, beta, cu_seqlens, S, T_total, state_pool, pool_size, slots,
                             has_initial, o, H, d_k, d_v, chunk, qkv_dtype, workspace, workspace_bytes,
                             stream) -> int:
    return lib().gdn_chunk_prefill_varlen(rule, q, k, v, g, beta, cu_seqlens, S, T_total, state_pool,
                                          pool_size, slots, has_initial, o, H, d_k, d_v, chunk, qkv_dtype,
                                          workspace, workspace_bytes, stream)


def gdn_chunk_prefill_varlen_workspace_size(cu_seqlens, S, H, d_k, d_v, chunk, qkv_dtype) -> int:
    return lib().gdn_chunk_prefill_varlen_workspace_size(cu_seqlens, S, H, d_k, d_v, chunk, qkv_dtype)


def gdn_prepare_decode_step(rule, xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, conv_state,
                            state, o, N, H, d_k, d_v, x_dtype, stream) -> int:
    return lib().gdn_prepare_decode_step(rule, xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias,
                                         conv_state, state, o, N, H, d_k, d_v, x_dtype, stream)


def gdn_prepare(xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, conv_state_in,
                conv_state_out, q, k, v, g, beta, B, T, H, d_k, d_v, x_dtype, stream) -> int:
    return lib().gdn_prepare(xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, conv_state_in,
                             conv_state_out, q, k, v, g, beta, B, T, H, d_k, d_v, x_dtype, stream)


def gdn_chunk_backward(rule, q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                       d_initial_state, B, T, H, d_k, d_v, qkv_dtype, workspace, workspace_bytes, stream) -> int:
    return lib().gdn_chunk_backward(rule, q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg,
                                    dbeta, d_initial_state, B, T, H, d_k, d_v, qkv_dtype, workspace,
                                    workspace_bytes, stream)


def gdn_chunk_backward_workspace_size(B, T, H, d_k, d_v, qkv_dtype) -> int:
    return lib().gdn_chunk_backward_workspace_size(B, T, H, d_k, d_v, qkv_dtype)


def gdn_prepare_varlen(xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, cu_seqlens, S, T_total,
                       conv_pool, pool_size, slots, has_initial, q, k, v, g, beta, H, d_k, d_v, x_dtype, workspace,
                       workspace_bytes, stream) -> int:
    return lib().gdn_prepare_varlen(xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, cu_seqlens, S,
                                    T_total, conv_pool, pool_size, slots, has_initial, q, k, v, g, beta, H, d_k, d_v,
                                    x_dtype, workspace, workspace_bytes, stream)


def gdn_prepare_varlen_workspace_size(S) -> int:
    return lib().gdn_prepare_varlen_workspace_size(S)


def gdn_prepare_chunk_prefill(rule, xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, conv_state_in,
                              conv_state_out, initial_state, o, final_state, B, T, H, d_k, d_v, chunk, x_dtype,
                              workspace, workspace_bytes, stream) -> int:
    return lib().gdn_prepare_chunk_prefill(rule, xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias,
                                           conv_state_in, conv_state_out, initial_state, o, final_state, B, T, H,
                                           d_k, d_v, chunk, x_dtype, workspace, workspace_bytes, stream)


def gdn_prepare_chunk_prefill_workspace_size(B, T, H, d_k, d_v, chunk, x_dtype) -> int:
    return lib().gdn_prepare_chunk_prefill_workspace_size(B, T, H, d_k, d_v, chunk, x_dtype)


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(status).decode()


def gdn_version() -> int:
    return lib().gdn_version()


# ---- torch helpers ------------------------------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, dtype=None, shape=None):
    """A GPU tensor (or None) of the given dtype and shape: the C ABI takes bare pointers, so a
    buffer of the wrong size would be read or written out of bounds."""
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream_of(stream, dev):
    """(raw stream handle, whether it was given by the caller)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream, False
    return stream, True


def _keep_until_done(tensors, stream, given):
    """Scratch allocated here is freed when the call returns; when the kernels run on a stream
    the caller named (not torch's current stream), tell torch's caching allocator that the
    memory is in use on that stream, so it is not handed out again before the kernels end."""
    if not given:
        return
    import torch
    ext = torch.cuda.ExternalStream(stream)
    for t in tensors:
        if t is not None:
            t.record_stream(ext)


def workspace_bytes(B, T, H, d_k, d_v, chunk, qkv_dtype) -> int:
    return int(gdn_chunk_prefill_workspace_size(B, T, H, d_k, d_v, chunk, qkv_dtype))


def chunk_prefill(q, k, v, g, beta, initial_state=None, chunk=64, *, out=None, final_state=None,
                  workspace=None, stream=None, rule=GDN_RULE_GATED_DELTA):
    """q, k [B,T,H,d_k]; v [B,T,H,d_v] (bf16 or fp32); g, beta [B,T,H] fp32;
    initial_state [B,H,d_k,d_v] fp32 or None.  Returns (o fp32 [B,T,H,d_v], final_state).
    ``final_state`` may be ``initial_state`` itself for in-place chaining.  ``rule`` is
    GDN_RULE_GATED_DELTA (default) or GDN_RULE_GATED_DECAY (no erase term)."""
    import torch
    B, T, H, d_k = q.shape
    d_v = v.shape[-1]
    dt = _dtype_code(q)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (B, T, H, d_k))
    _check(v, "v", q.dtype, (B, T, H, d_v))
    _check(g, "g", torch.float32, (B, T, H))
    _check(beta, "beta", torch.float32, (B, T, H))
    _check(initial_state, "initial_state", torch.float32, (B, H, d_k, d_v))
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, d_v), device=dev, dtype=torch.float32)
    if final_state is None:
        final_state = torch.empty((B, H, d_k, d_v), device=dev, dtype=torch.float32)
    _check(out, "out", torch.float32, (B, T, H, d_v))
    _check(final_state, "final_state", torch.float32, (B, H, d_k, d_v))
    need = workspace_bytes(B, T, H, d_k, d_v, chunk, dt)
    own_ws = workspace is None and need > 0
    if own_ws:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream, given = _stream_of(stream, dev)
    st = gdn_chunk_prefill_rule(rule, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(initial_state), _ptr(out), _ptr(final_state), B, T, H, d_k, d_v,
                                chunk, dt, _ptr(workspace), ws_bytes, stream)
    if st != 0:
        raise GdnError(st, "gdn_chunk_prefill_rule")
    _keep_until_done([workspace] if own_ws else [], stream, given)
    return out, final_state


def decode_step(q, k, v, g, beta, state, *, out=None, stream=None, rule=GDN_RULE_GATED_DELTA):
    """q, k [N,H,d_k]; v [N,H,d_v]; g, beta [N,H] fp32; state [N,H,d_k,d_v] fp32
    (updated in place).  Returns o fp32 [N,H,d_v].  ``rule`` as for chunk_prefill."""
    import torch
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    dt = _dtype_code(q)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (N, H, d_k))
    _check(v, "v", q.dtype, (N, H, d_v))
    _check(g, "g", torch.float32, (N, H))
    _check(beta, "beta", torch.float32, (N, H))
    _check(state, "state", torch.float32, (N, H, d_k, d_v))
    if out is None:
        out = torch.empty((N, H, d_v), device=q.device, dtype=torch.float32)
    _check(out, "out", torch.float32, (N, H, d_v))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = gdn_decode_step_rule(rule, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                              _ptr(out), N, H, d_k, d_v, dt, stream)
    if st != 0:
        raise GdnError(st, "gdn_decode_step_rule")
    return out


def decode_step_slots(q, k, v, g, beta, state_pool, slots, *, out=None, stream=None,
                      rule=GDN_RULE_GATED_DELTA):
    """q, k [N,H,d_k]; v [N,H,d_v]; g, beta [N,H] fp32; state_pool [P,H,d_k,d_v] fp32;
    slots [N] int32 on the GPU: sequence n updates state_pool[slots[n]] in place; a slot
    outside [0, P) is padding (zero output, no state touched).  Returns o fp32 [N,H,d_v]."""
    import torch
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    dt = _dtype_code(q)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (N, H, d_k))
    _check(v, "v", q.dtype, (N, H, d_v))
    _check(g, "g", torch.float32, (N, H))
    _check(beta, "beta", torch.float32, (N, H))
    _check(state_pool, "state_pool", torch.float32)
    if state_pool is not None:
        _check(state_pool, "state_pool", torch.float32, (state_pool.shape[0], H, d_k, d_v))
    _check(slots, "slots", torch.int32, (N,))
    if out is None:
        out = torch.empty((N, H, d_v), device=q.device, dtype=torch.float32)
    _check(out, "out", torch.float32, (N, H, d_v))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = gdn_decode_step_slots(rule, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                               _ptr(slots), state_pool.shape[0], _ptr(out), N, H, d_k, d_v, dt, stream)
    if st != 0:
        raise GdnError(st, "gdn_decode_step_slots")
    return out


def prepare_decode_step(xq, xk, xv, conv_weight, a_raw, b_raw, conv_state, state, *, decay_rate=None,
                        gate_bias=None, out=None, stream=None, rule=GDN_RULE_GATED_DELTA):
    """One token per sequence from the raw projections: xq, xk [N,H,d_k], xv [N,H,d_v] (bf16 or fp32);
    conv_weight [H*(2 d_k + d_v), 4] fp32; a_raw, b_raw [N,H] fp32; conv_state [N, H*(2 d_k + d_v), 3]
    fp32 and state [N,H,d_k,d_v] fp32, both updated in place; decay_rate, gate_bias [H] fp32 or None.
    Returns o fp32 [N,H,d_v] (prepare with T = 1, then decode_step, in one launch)."""
    import torch
    N, H, d_k = xq.shape
    d_v = xv.shape[-1]
    dt = _dtype_code(xq)
    C = H * (2 * d_k + d_v)
    _check(xq, "xq", xq.dtype)
    _check(xk, "xk", xq.dtype, (N, H, d_k))
    _check(xv, "xv", xq.dtype, (N, H, d_v))
    for t, n, shp in ((conv_weight, "conv_weight", (C, 4)), (a_raw, "a_raw", (N, H)), (b_raw, "b_raw", (N, H)),
                      (decay_rate, "decay_rate", (H,)), (gate_bias, "gate_bias", (H,)),
                      (conv_state, "conv_state", (N, C, 3)), (state, "state", (N, H, d_k, d_v))):
        _check(t, n, torch.float32, shp)
    if out is None:
        out = torch.empty((N, H, d_v), device=xq.device, dtype=torch.float32)
    _check(out, "out", torch.float32, (N, H, d_v))
    if stream is None:
        stream = torch.cuda.current_stream(xq.device).cuda_stream
    st = gdn_prepare_decode_step(rule, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_weight), _ptr(a_raw), _ptr(b_raw),
                                 _ptr(decay_rate), _ptr(gate_bias), _ptr(conv_state), _ptr(state), _ptr(out),
                                 N, H, d_k, d_v, dt, stream)
    if st != 0:
        raise GdnError(st, "gdn_prepare_decode_step")
    return out


def prepare(xq, xk, xv, conv_weight, a_raw, b_raw, *, decay_rate=None, gate_bias=None, conv_state=None,
            conv_state_out=None, outs=None, stream=None):
    """Input preparation ahead of the mixer.  xq, xk [B,T,H,d_k]; xv [B,T,H,d_v] (bf16 or fp32);
    conv_weight [H*(2 d_k + d_v), 4] fp32; a_raw, b_raw [B,T,H] fp32; decay_rate, gate_bias [H] fp32
    or None; conv_state [B, H*(2 d_k + d_v), 3] fp32 or None (zeros).  conv_state_out receives the
    carried state (pass conv_state itself to update it in place; None = not kept).
    Returns (q, k, v, g, beta) ready for chunk_prefill / decode_step."""
    import torch
    B, T, H, d_k = xq.shape
    d_v = xv.shape[-1]
    dt = _dtype_code(xq)
    C = H * (2 * d_k + d_v)
    _check(xq, "xq", xq.dtype)
    _check(xk, "xk", xq.dtype, (B, T, H, d_k))
    _check(xv, "xv", xq.dtype, (B, T, H, d_v))
    for t, n, shp in ((conv_weight, "conv_weight", (C, 4)), (a_raw, "a_raw", (B, T, H)), (b_raw, "b_raw", (B, T, H)),
                      (decay_rate, "decay_rate", (H,)), (gate_bias, "gate_bias", (H,)),
                      (conv_state, "conv_state", (B, C, 3)), (conv_state_out, "conv_state_out", (B, C, 3))):
        _check(t, n, torch.float32, shp)
    dev = xq.device
    if outs is None:
        outs = (torch.empty_like(xq), torch.empty_like(xk), torch.empty_like(xv),
                torch.empty((B, T, H), device=dev, dtype=torch.float32),
                torch.empty((B, T, H), device=dev, dtype=torch.float32))
    q, k, v, g, beta = outs
    _check(q, "q", xq.dtype, (B, T, H, d_k))
    _check(k, "k", xq.dtype, (B, T, H, d_k))
    _check(v, "v", xq.dtype, (B, T, H, d_v))
    _check(g, "g", torch.float32, (B, T, H))
    _check(beta, "beta", torch.float32, (B, T, H))
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = gdn_prepare(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_weight), _ptr(a_raw), _ptr(b_raw), _ptr(decay_rate),
                     _ptr(gate_bias), _ptr(conv_state), _ptr(conv_state_out), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                     _ptr(beta), B, T, H, d_k, d_v, dt, stream)
    if st != 0:
        raise GdnError(st, "gdn_prepare")
    return q, k, v, g, beta


def prepare_chunk_prefill(xq, xk, xv, conv_weight, a_raw, b_raw, initial_state=None, *, decay_rate=None,
                          gate_bias=None, conv_state=None, conv_state_out=None, chunk=64, out=None, final_state=None,
                          workspace=None, stream=None, rule=GDN_RULE_GATED_DELTA):
    """The preparation ahead of the mixer and the prefill in one pass (prepare() then chunk_prefill(),
    without the prepared q, k, v, g, beta in device memory).  xq, xk [B,T,H,d_k], xv [B,T,H,d_v] bf16;
    conv_weight [H*(2 d_k + d_v), 4]; a_raw, b_raw [B,T,H]; decay_rate, gate_bias [H] or None; conv_state
    [B, H*(2 d_k + d_v), 3] or None (zeros); conv_state_out receives the carried window (pass conv_state
    itself to update it in place); initial_state [B,H,d_k,d_v] or None.  Returns (o, final_state)."""
    import torch
    B, T, H, d_k = xq.shape
    d_v = xv.shape[-1]
    dt = _dtype_code(xq)
    C = H * (2 * d_k + d_v)
    _check(xq, "xq", xq.dtype)
    _check(xk, "xk", xq.dtype, (B, T, H, d_k))
    _check(xv, "xv", xq.dtype, (B, T, H, d_v))
    for t, n, shp in ((conv_weight, "conv_weight", (C, 4)), (a_raw, "a_raw", (B, T, H)), (b_raw, "b_raw", (B, T, H)),
                      (decay_rate, "decay_rate", (H,)), (gate_bias, "gate_bias", (H,)),
                      (conv_state, "conv_state", (B, C, 3)), (conv_state_out, "conv_state_out", (B, C, 3)),
                      (initial_state, "initial_state", (B, H, d_k, d_v))):
        _check(t, n, torch.float32, shp)
    dev = xq.device
    if out is None:
        out = torch.empty((B, T, H, d_v), device=dev, dtype=torch.float32)
    if final_state is None:
        final_state = torch.empty((B, H, d_k, d_v), device=dev, dtype=torch.float32)
    _check(out, "out", torch.float32, (B, T, H, d_v))
    _check(final_state, "final_state", torch.float32, (B, H, d_k, d_v))
    need = int(gdn_prepare_chunk_prefill_workspace_size(B, T, H, d_k, d_v, chunk, dt))
    own_ws = workspace is None and need > 0
    if own_ws:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream, given = _stream_of(stream, dev)
    st = gdn_prepare_chunk_prefill(rule, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_weight), _ptr(a_raw), _ptr(b_raw),
                                   _ptr(decay_rate), _ptr(gate_bias), _ptr(conv_state), _ptr(conv_state_out),
                                   _ptr(initial_state), _ptr(out), _ptr(final_state), B, T, H, d_k, d_v, chunk, dt,
                                   _ptr(workspace), ws_bytes, stream)
    if st != 0:
        raise GdnError(st, "gdn_prepare_chunk_prefill")
    _keep_until_done([workspace] if own_ws else [], stream, given)
    return out, final_state


def chunk_backward(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None, *, want_d_initial=True,
                   outs=None, workspace=None, stream=None, rule=GDN_RULE_GATED_DELTA):
    """Gradients of one prefill call for L = <d_o, o> + <d_final_state, S_T>.  Inputs as for
    chunk_prefill (bf16 or fp32 q/k/v, d_k = d_v = 64 or 128); d_o [B,T,H,d_v] fp32; d_final_state [B,H,d_k,d_v]
    fp32 or None.  Returns (dq, dk, dv, dg, dbeta, d_initial_state or None), all fp32."""
    import torch
    B, T, H, d_k = q.shape
    d_v = v.shape[-1]
    dt = _dtype_code(q)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (B, T, H, d_k))
    _check(v, "v", q.dtype, (B, T, H, d_v))
    for t, n, shp in ((g, "g", (B, T, H)), (beta, "beta", (B, T, H)), (d_o, "d_o", (B, T, H, d_v)),
                      (initial_state, "initial_state", (B, H, d_k, d_v)),
                      (d_final_state, "d_final_state", (B, H, d_k, d_v))):
        _check(t, n, torch.float32, shp)
    dev = q.device
    if outs is None:
        f32 = dict(device=dev, dtype=torch.float32)
        outs = (torch.empty((B, T, H, d_k), **f32), torch.empty((B, T, H, d_k), **f32),
                torch.empty((B, T, H, d_v), **f32), torch.empty((B, T, H), **f32), torch.empty((B, T, H), **f32),
                torch.empty((B, H, d_k, d_v), **f32) if want_d_initial else None)
    shapes = ((B, T, H, d_k), (B, T, H, d_k), (B, T, H, d_v), (B, T, H), (B, T, H), (B, H, d_k, d_v))
    for t, n, shp in zip(outs, ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state"), shapes):
        _check(t, n, torch.float32, shp)
    need = int(gdn_chunk_backward_workspace_size(B, T, H, d_k, d_v, dt))
    own_ws = workspace is None and need > 0
    if own_ws:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream, given = _stream_of(stream, dev)
    st = gdn_chunk_backward(rule, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(d_o),
                            _ptr(d_final_state), *[_ptr(t) for t in outs], B, T, H, d_k, d_v, dt,
                            _ptr(workspace), ws_bytes, stream)
    if st != 0:
        raise GdnError(st, "gdn_chunk_backward")
    _keep_until_done([workspace] if own_ws else [], stream, given)
    return outs


def backward_workspace_bytes(B, T, H, d_k, d_v, qkv_dtype) -> int:
    return int(gdn_chunk_backward_workspace_size(B, T, H, d_k, d_v, qkv_dtype))


def _host_i32(x):
    """A host int32 array (numpy) from a list, numpy array or CPU tensor, or None."""
    import numpy as np
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.device.type != "cpu":
                raise TypeError("cu_seqlens, slots and has_initial are host arrays")
            x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _np_ptr(a):
    return None if a is None else a.ctypes.data


def varlen_workspace_bytes(cu_seqlens, H, d_k, d_v, chunk, qkv_dtype) -> int:
    cu = _host_i32(cu_seqlens)
    return int(gdn_chunk_prefill_varlen_workspace_size(_np_ptr(cu), len(cu) - 1, H, d_k, d_v, chunk,
                                                       qkv_dtype))


def prepare_varlen(xq, xk, xv, conv_weight, a_raw, b_raw, cu_seqlens, conv_pool, slots=None, has_initial=None, *,
                   decay_rate=None, gate_bias=None, outs=None, workspace=None, stream=None):
    """Input preparation of packed sequences: xq, xk [T,H,d_k]; xv [T,H,d_v]; a_raw, b_raw [T,H] fp32;
    cu_seqlens host int32 [S+1]; conv_pool [P, H*(2 d_k + d_v), 3] fp32 (sequence s starts from and ends in
    slot slots[s], slot s when slots is None; -1 = from zeros, state dropped); has_initial host [S].
    Returns (q, k, v, g, beta) packed like the inputs."""
    import torch
    T, H, d_k = xq.shape
    d_v = xv.shape[-1]
    dt = _dtype_code(xq)
    C = H * (2 * d_k + d_v)
    _check(xq, "xq", xq.dtype)
    _check(xk, "xk", xq.dtype, (T, H, d_k))
    _check(xv, "xv", xq.dtype, (T, H, d_v))
    for t, n, shp in ((conv_weight, "conv_weight", (C, 4)), (a_raw, "a_raw", (T, H)), (b_raw, "b_raw", (T, H)),
                      (decay_rate, "decay_rate", (H,)), (gate_bias, "gate_bias", (H,))):
        _check(t, n, torch.float32, shp)
    _check(conv_pool, "conv_pool", torch.float32)
    if conv_pool is not None:
        _check(conv_pool, "conv_pool", torch.float32, (conv_pool.shape[0], C, 3))
    cu, sl, hi = _host_i32(cu_seqlens), _host_i32(slots), _host_i32(has_initial)
    S = len(cu) - 1
    dev = xq.device
    if outs is None:
        outs = (torch.empty_like(xq), torch.empty_like(xk), torch.empty_like(xv),
                torch.empty((T, H), device=dev, dtype=torch.float32), torch.empty((T, H), device=dev, dtype=torch.float32))
    for t, n, dtp, shp in zip(outs, ("q", "k", "v", "g", "beta"), (xq.dtype, xq.dtype, xq.dtype, torch.float32,
                                                                  torch.float32),
                              ((T, H, d_k), (T, H, d_k), (T, H, d_v), (T, H), (T, H))):
        _check(t, n, dtp, shp)
    need = int(gdn_prepare_varlen_workspace_size(S))
    own_ws = workspace is None and need > 0
    if own_ws:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream, given = _stream_of(stream, dev)
    pool_size = 0 if conv_pool is None else conv_pool.shape[0]
    st = gdn_prepare_varlen(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_weight), _ptr(a_raw), _ptr(b_raw),
                            _ptr(decay_rate), _ptr(gate_bias), _np_ptr(cu), S, T, _ptr(conv_pool), pool_size,
                            _np_ptr(sl), _np_ptr(hi), *[_ptr(t) for t in outs], H, d_k, d_v, dt, _ptr(workspace),
                            ws_bytes, stream)
    if st != 0:
        raise GdnError(st, "gdn_prepare_varlen")
    _keep_until_done([workspace] if own_ws else [], stream, given)
    return outs


def chunk_prefill_varlen(q, k, v, g, beta, cu_seqlens, state_pool, slots=None, has_initial=None, chunk=64,
                         *, out=None, workspace=None, stream=None, rule=GDN_RULE_GATED_DELTA):
    """Packed sequences: q, k [T,H,d_k]; v [T,H,d_v] bf16; g, beta [T,H] fp32; cu_seqlens host int32
    [S+1]; state_pool [P,H,d_k,d_v] fp32 (sequence s starts from and ends in slot slots[s], slot s when
    slots is None; -1 = from zeros, final state dropped); has_initial host [S] (0 = start from zeros).
    Returns o fp32 [T,H,d_v]; final states are written into the pool."""
    import torch
    T, H, d_k = q.shape
    d_v = v.shape[-1]
    dt = _dtype_code(q)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (T, H, d_k))
    _check(v, "v", q.dtype, (T, H, d_v))
    _check(g, "g", torch.float32, (T, H))
    _check(beta, "beta", torch.float32, (T, H))
    _check(state_pool, "state_pool", torch.float32)
    if state_pool is not None:
        _check(state_pool, "state_pool", torch.float32, (state_pool.shape[0], H, d_k, d_v))
    cu, sl, hi = _host_i32(cu_seqlens), _host_i32(slots), _host_i32(has_initial)
    S = len(cu) - 1
    if out is None:
        out = torch.empty((T, H, d_v), device=q.device, dtype=torch.float32)
    _check(out, "out", torch.float32, (T, H, d_v))
    need = int(gdn_chunk_prefill_varlen_workspace_size(_np_ptr(cu), S, H, d_k, d_v, chunk, dt))
    own_ws = workspace is None and need > 0
    if own_ws:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream, given = _stream_of(stream, q.device)
    pool_size = 0 if state_pool is None else state_pool.shape[0]
    st = gdn_chunk_prefill_varlen(rule, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _np_ptr(cu), S, T,
                                  _ptr(state_pool), pool_size, _np_ptr(sl), _np_ptr(hi), _ptr(out), H, d_k, d_v,
                                  chunk, dt, _ptr(workspace), ws_bytes, stream)
    if st != 0:
        raise GdnError(st, "gdn_chunk_prefill_varlen")
    _keep_until_done([workspace] if own_ws else [], stream, given)
    return out


__all__ = ["EXPORTS", "GDN_F32", "GDN_BF16", "GDN_RULE_GATED_DELTA", "GDN_RULE_GATED_DECAY", "GdnError",
           "lib", "gdn_chunk_prefill", "gdn_chunk_prefill_rule", "gdn_chunk_prefill_workspace_size",
           "gdn_chunk_prefill_noalloc",
           "gdn_decode_step", "gdn_decode_step_rule", "gdn_status_string", "gdn_version",
           "gdn_decode_step_slots", "gdn_chunk_prefill_varlen", "gdn_chunk_prefill_varlen_workspace_size",
           "chunk_prefill", "chunk_prefill_varlen", "decode_step", "decode_step_slots", "workspace_bytes",
           "varlen_workspace_bytes", "gdn_prepare", "prepare", "gdn_chunk_backward",
           "gdn_chunk_backward_workspace_size", "chunk_backward", "backward_workspace_bytes", "gdn_prepare_varlen",
           "gdn_prepare_varlen_workspace_size", "prepare_varlen", "gdn_prepare_decode_step", "prepare_decode_step",
           "gdn_prepare_chunk_prefill", "gdn_prepare_chunk_prefill_workspace_size", "prepare_chunk_prefill"]
