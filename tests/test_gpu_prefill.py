"""GPU parity of gdn_chunk_prefill against the fp64 oracle (MI355X only).

Small shapes are compared element by element over every output and state
entry; the full-size workloads (B=4/H=32/T=8192 and B=1/H=32/T=65536 with
d=64, and the 32-call 2M-token chain with H=24, d=128) are run exactly as the
benchmark runs them and compared on sampled value rows, which the oracle
evaluates one row at a time (value rows of the state evolve independently).
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import hybrid_linear_attention_gated_amd as gdn
from parity import TOL, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def tol_of(dtype):
    return TOL["f32"] if dtype == torch.float32 else TOL["bf16"]


def inputs(B, T, H, dk, dv, dtype, s0=True, gate="primary", shift=3.0, call=0, wid=50):
    return gi.prefill_inputs(B, T, H, dk, dv, wid=wid, call=call, qkv_dtype=dtype, gate=gate,
                             gate_shift=shift, s0=s0, device=DEV)


def run_gpu(d, chunk):
    o, sf = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk=chunk)
    torch.cuda.synchronize()
    return o.cpu().numpy(), sf.cpu().numpy()


def run_oracle(orc, d, rows=None):
    return orc.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], rows=rows)


def check(orc, d, chunk, tol, what, rows=None):
    print(f"[case] {what} chunk={chunk}", flush=True)
    o, sf = run_gpu(d, chunk)
    ro, rs = run_oracle(orc, d, rows)
    assert_parity(o, ro, tol, what + " outputs")
    assert_parity(sf, rs, tol, what + " final state")
    return o, sf


# --- small shapes: every element --------------------------------------------------------

def test_tiny_fp32_workload(orc):
    """B=1, H=2, T=64, d=16, all fp32, chunk 16, zero start state."""
    d = gi.workload_inputs("tiny", device=DEV)
    check(orc, d, 16, TOL["f32"], "tiny fp32")


@pytest.mark.parametrize("gate", ["primary", "literal"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("chunk", [32, 64])
def test_bf16_mfma_path(orc, gate, dk, dv, chunk):
    """Several chunks plus a ragged tail, nonzero start state."""
    d = inputs(2, 3 * chunk + 7, 3, dk, dv, torch.bfloat16, gate=gate)
    check(orc, d, chunk, TOL["bf16"], f"bf16 dk={dk} dv={dv} gate={gate}")


@pytest.mark.parametrize("gate", ["primary", "literal"])
@pytest.mark.parametrize("dk,dv,chunk,T,s0", [
    (64, 64, 64, 2560, True), (64, 64, 64, 2547, False), (128, 128, 64, 2560, True),
    (64, 128, 32, 2600, True), (128, 64, 64, 4096, True),
    # two and three pieces: the shortest chains (one and two map steps)
    (64, 64, 64, 1100, True), (128, 128, 64, 1600, True), (64, 64, 64, 1536, False)])
def test_bf16_sequence_pieces(orc, gate, dk, dv, chunk, T, s0):
    """Long sequences on few heads are split into pieces (piece maps, then a chained
    start state per piece): every element, ragged tails included."""
    d = inputs(1, T, 2, dk, dv, torch.bfloat16, s0=s0, gate=gate)
    check(orc, d, chunk, TOL["bf16"], f"pieces T={T} dk={dk} dv={dv} gate={gate}")


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
def test_map_drops_then_expanding_chunk(orc, dk, dv):
    """The map pass drops an identity slice once it is below 2^-32 only while no token of the
    piece so far can expand the map; a later chunk that can (b |k|^2 > 2) makes it recompute the
    piece's map from its first chunk with no drops.  Even 32-token chunks decay hard (g = -1.1:
    their maps fall far below 2^-32); odd ones have b = 1 and |k|^2 near 2.2 (the token's map
    I - b k k^T has an eigenvalue near -1.2).  Pieces of nine chunks start on even and odd chunks
    in turn: the first drop and then restart, the others stop dropping before any drop.  Every
    element against the oracle."""
    d = inputs(1, 4096 + 19, 2, dk, dv, torch.bfloat16)
    odd = ((torch.arange(d["g"].shape[1], device=DEV) // 32) % 2 == 1)[None, :, None]
    d["g"] = torch.where(odd, d["g"], torch.full_like(d["g"], -1.1))
    d["beta"] = torch.where(odd, torch.ones_like(d["beta"]), d["beta"])
    d["k"] = torch.where(odd[..., None], (d["k"].float() * 2.2 ** 0.5).to(torch.bfloat16), d["k"])
    check(orc, d, 64, TOL["bf16"], f"map drops then expanding keys dk={dk} dv={dv}")


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 64), (64, 16), (64, 64)])
def test_bf16_chunk16_and_small_heads(orc, dk, dv):
    d = inputs(1, 70, 2, dk, dv, torch.bfloat16)
    check(orc, d, 16, TOL["bf16"], f"bf16 small dk={dk} dv={dv}")


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 64), (128, 128), (16, 128)])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fp32_path(orc, dk, dv, chunk):
    d = inputs(2, 2 * chunk + 5, 2, dk, dv, torch.float32)
    check(orc, d, chunk, TOL["f32"], f"fp32 dk={dk} dv={dv}")


def test_chunk_sizes_agree(orc):
    """chunk 16, 32 and 64 all match the same oracle result."""
    d = inputs(1, 300, 4, 64, 64, torch.bfloat16)
    ro, rs = run_oracle(orc, d)
    for chunk in (16, 32, 64):
        o, sf = run_gpu(d, chunk)
        assert_parity(o, ro, TOL["bf16"], f"chunk {chunk} outputs")
        assert_parity(sf, rs, TOL["bf16"], f"chunk {chunk} state")


@pytest.mark.parametrize("T", [1, 2, 63, 65])
@pytest.mark.parametrize("d_head", [64, 128])
def test_short_and_ragged_lengths(orc, T, d_head):
    """Sequences shorter than a chunk or one token past it (128-wide heads run eight-wavefront
    workgroups)."""
    d = inputs(2, T, 2, d_head, d_head, torch.bfloat16)
    check(orc, d, 64, TOL["bf16"], f"T={T} d={d_head}")


def test_zero_length_copies_the_state():
    d = inputs(1, 0, 2, 64, 64, torch.bfloat16)
    o, sf = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    _, sz = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(sf, d["s0"]) and torch.all(sz == 0)


# --- special cases of the rule, on the GPU ------------------------------------------------------

def test_no_write_no_decay_keeps_state():
    """b = 0, a = 1: the state passes through and o_t = S0 q_t / sqrt(d_k)."""
    d = inputs(1, 130, 2, 64, 64, torch.bfloat16)
    d["beta"].zero_()
    d["g"].zero_()
    o, sf = run_gpu(d, 64)
    s0 = d["s0"].cpu().double().numpy()
    expect = np.einsum("bthj,bhji->bthi", d["q"].double().cpu().numpy(), s0) / 8.0
    assert_parity(sf, s0, 1e-5, "state unchanged")
    assert_parity(o, expect, TOL["bf16"], "o = S0 q / sqrt(d_k)")


def test_vanishing_gate_resets_state():
    """a -> 0 (g = -200): S_t = b_t v_t k_t^T and o_t = b_t (k_t . q_t) v_t / sqrt(d_k)."""
    d = inputs(1, 100, 2, 64, 64, torch.bfloat16)
    d["g"].fill_(-200.0)
    o, sf = run_gpu(d, 64)
    q, k, v = (d[x].double().cpu().numpy() for x in ("q", "k", "v"))
    b = d["beta"].double().cpu().numpy()
    expect = (b * np.einsum("bthj,bthj->bth", k, q))[..., None] * v / 8.0
    assert_parity(o, expect, TOL["bf16"], "rank-one readout")
    last = b[:, -1, :, None, None] * np.einsum("bhj,bhi->bhji", k[:, -1], v[:, -1])
    assert_parity(sf, last, TOL["bf16"], "rank-one state")


def test_orthonormal_keys_overwrite():
    """b = 1, a = 1, orthonormal keys: S k_j returns the latest value written under k_j."""
    dk = dv = 64
    rng = np.random.default_rng(3)
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Q.T  # 64 orthonormal keys
    order = np.concatenate([np.arange(64), [5, 17, 5]])
    T = len(order)
    vals = rng.standard_normal((T, dv))
    k = torch.tensor(keys[order][None, :, None, :], dtype=torch.float32, device=DEV)
    v = torch.tensor(vals[None, :, None, :], dtype=torch.float32, device=DEV)
    q = k.clone()
    g = torch.zeros(1, T, 1, device=DEV)
    b = torch.ones(1, T, 1, device=DEV)
    _, sf = gdn.chunk_prefill(q, k, v, g, b, None, chunk=32)
    torch.cuda.synchronize()
    S = sf[0, 0].double().cpu().numpy().T  # [dv, dk]
    latest = {}
    for t, j in enumerate(order):
        latest[j] = vals[t]
    got = np.stack([S @ keys[j] for j in range(64)])
    expect = np.stack([latest[j] for j in range(64)])
    assert_parity(got, expect, TOL["f32"], "exact retrieval after overwrite")


# --- chaining, decode equivalence, determinism ---------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_chained_calls_equal_one_call(orc, dtype):
    """T tokens in one call vs two calls through the carried state (split not chunk-aligned),
    the second call updating the state in place."""
    d = inputs(2, 300, 3, 64, 64, dtype)
    o_full, s_full = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    T1 = 101
    part = lambda x, a, b: x[:, a:b].contiguous()
    state = d["s0"].clone()
    o1, _ = gdn.chunk_prefill(*(part(d[x], 0, T1) for x in ("q", "k", "v", "g", "beta")), state,
                              final_state=state)
    o2, _ = gdn.chunk_prefill(*(part(d[x], T1, 300) for x in ("q", "k", "v", "g", "beta")), state,
                              final_state=state)
    torch.cuda.synchronize()
    o_chain = torch.cat([o1, o2], dim=1).cpu().numpy()
    ro, rs = run_oracle(orc, d)
    tol = tol_of(dtype)
    assert_parity(o_chain, ro, tol, "chained outputs")
    assert_parity(state.cpu().numpy(), rs, tol, "chained final state")
    assert_parity(o_chain, o_full.cpu().numpy(), tol, "chained vs one call")


def test_decode_steps_equal_prefill(orc):
    """16 decode steps equal one prefill over the same 16 tokens."""
    N, H, d = 8, 4, 64
    x = inputs(N, 16, H, d, d, torch.bfloat16)
    o_pre, s_pre = gdn.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], chunk=64)
    state = x["s0"].clone()
    outs = [gdn.decode_step(*(x[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")), state)
            for t in range(16)]
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1).cpu().numpy()
    ro, rs = run_oracle(orc, x)
    assert_parity(o_dec, ro, TOL["bf16"], "decode x16 outputs")
    assert_parity(o_pre.cpu().numpy(), ro, TOL["bf16"], "prefill outputs")
    assert_parity(state.cpu().numpy(), s_pre.cpu().numpy(), TOL["bf16"], "decode vs prefill state")


def test_prefill_is_deterministic():
    d = inputs(1, 1000, 8, 64, 64, torch.bfloat16)
    a = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    b = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_prefill_guard_regions_untouched():
    B, T, H, dk = 1, 200, 3, 64
    pad = 4096
    d = inputs(B, T, H, dk, dk, torch.bfloat16)
    obuf = torch.full((pad + B * T * H * dk + pad,), 9.5, device=DEV)
    sbuf = torch.full((pad + B * H * dk * dk + pad,), -1.25, device=DEV)
    n_ws = gdn.workspace_bytes(B, T, H, dk, dk, 64, gdn.GDN_BF16)
    wbuf = torch.full((pad + n_ws + pad,), 77, dtype=torch.uint8, device=DEV)
    out = obuf[pad:pad + B * T * H * dk].view(B, T, H, dk)
    fin = sbuf[pad:pad + B * H * dk * dk].view(B, H, dk, dk)
    gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], out=out, final_state=fin,
                      workspace=wbuf[pad:pad + n_ws])
    torch.cuda.synchronize()
    for buf, val in ((obuf, 9.5), (sbuf, -1.25), (wbuf, 77)):
        assert torch.all(buf[:pad] == val) and torch.all(buf[-pad:] == val)


def test_prefill_error_has_no_side_effect():
    B, T, H, d = 1, 2560, 2, 64  # long enough to be split into pieces: needs workspace
    assert gdn.workspace_bytes(B, T, H, d, d, 64, gdn.GDN_BF16) > 0
    x = inputs(B, T, H, d, d, torch.bfloat16)
    o = torch.full((B, T, H, d), 5.0, device=DEV)
    sf = torch.full((B, H, d, d), 6.0, device=DEV)
    st = gdn.gdn_chunk_prefill(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(),
                               x["g"].data_ptr(), x["beta"].data_ptr(), x["s0"].data_ptr(),
                               o.data_ptr(), sf.data_ptr(), B, T, H, d, d, 64, gdn.GDN_BF16,
                               None, 0, None)
    torch.cuda.synchronize()
    assert st == 6  # workspace missing
    assert torch.all(o == 5.0) and torch.all(sf == 6.0)


# --- full-size workloads, as the benchmark runs them ---------------------------------------

# one value row in every 16-column slice of the state (each slice is a wavefront's share)
ROWS = [0, 21, 38, 63]


def test_workload_1b_8k(orc):
    """B=4, H=32, T=8192, d=64, chunk 64, zero start state: every element."""
    d = gi.workload_inputs("1b_8k", device=DEV)
    check(orc, d, 64, TOL["bf16"], "1b_8k (B=4 H=32 T=8192)")


@pytest.mark.parametrize("gate", ["primary", "literal"])
def test_workload_1b_64k(orc, gate):
    """B=1, H=32, T=65536, d=64, chunk 64, start state carried in: sampled value rows."""
    d = gi.workload_inputs("1b_64k", gate=gate, device=DEV)
    print(f"[case] 1b_64k gate={gate}", flush=True)
    o, sf = run_gpu(d, 64)
    ro, rs = run_oracle(orc, d, rows=ROWS)
    assert_parity(o[..., ROWS], ro[..., ROWS], TOL["bf16"], f"1b_64k {gate} outputs (rows {ROWS})")
    assert_parity(sf[..., ROWS], rs[..., ROWS], TOL["bf16"], f"1b_64k {gate} state (rows {ROWS})")


def test_workload_3b_2m_chain(orc):
    """H=24, d=128: 32 chained calls of T=65536 through the carried state (2M tokens),
    compared after every call on sampled value rows against an oracle chaining its own state."""
    w = gi.WORKLOADS["3b_2m"]
    rows = [3, 17, 34, 50, 77, 85, 102, 127]  # one per 16-column slice (eight wavefronts)
    state = torch.zeros(1, w.H, w.dk, w.dv, device=DEV)
    ws = torch.empty(gdn.workspace_bytes(1, w.T, w.H, w.dk, w.dv, 64, gdn.GDN_BF16), dtype=torch.uint8,
                     device=DEV)
    ref_state = np.zeros((1, w.H, w.dk, w.dv))
    worst = 0.0
    for call in range(w.calls):
        d = gi.workload_inputs("3b_2m", call=call, device=DEV)
        o, _ = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], state, chunk=64,
                                 final_state=state, workspace=ws)
        torch.cuda.synchronize()
        ro, rs = orc.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], ref_state, rows=rows)
        ref_state[..., rows] = rs[..., rows]
        e1 = assert_parity(o.cpu().numpy()[..., rows], ro[..., rows], TOL["bf16"], f"3b_2m call {call} outputs")
        e2 = assert_parity(state.cpu().numpy()[..., rows], ref_state[..., rows], TOL["bf16"],
                           f"3b_2m call {call} state")
        worst = max(worst, e1, e2)
    print(f"[parity] 3b_2m worst over 32 calls: {worst:.3e}", flush=True)


def test_ragged_64k_plus_one(orc):
    """T = 65537 (a partial last chunk of one token) with a start state, as one call at the
    64K layer shape (B=1, H=32, d=64): every 16-column slice sampled."""
    d = inputs(1, 65537, 32, 64, 64, torch.bfloat16, s0=True, wid=57)
    print("[case] ragged B=1 H=32 T=65537", flush=True)
    o, sf = run_gpu(d, 64)
    ro, rs = run_oracle(orc, d, rows=ROWS)
    assert_parity(o[..., ROWS], ro[..., ROWS], TOL["bf16"], f"T=65537 outputs (rows {ROWS})")
    assert_parity(sf[..., ROWS], rs[..., ROWS], TOL["bf16"], f"T=65537 state (rows {ROWS})")
