"""GPU parity of the gradients of the chunked prefill (MI355X only).

Every gradient (dq, dk, dv, dg, dbeta, d_initial_state) of the HIP path is compared element by
element with the fp64 token-by-token adjoint of the oracle on the same seeded inputs (q, k, v
stored as bf16, so both sides see the same values), within the bf16-input tolerance of the
forward (max |err| <= 2e-2 RMS of the oracle's tensor; 1e-4 for fp32 q/k/v).  Cases: ragged lengths, several forward
pieces, both rules, with and without start state and final-state gradient, T = 0 and 1, the
full 1b_8k training shape, and 128-wide heads (the 3B-shaped layers) on ragged, multi-piece and
two-level-scan sequences and on sampled heads of a 24-head 8K call."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import hybrid_linear_attention_gated_amd as gdn
import oracle
from parity import TOL, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ORULE = {gdn.GDN_RULE_GATED_DELTA: oracle.GATED_DELTA, gdn.GDN_RULE_GATED_DECAY: oracle.GATED_DECAY}


def grad_inputs(B, T, H, d, wid, s0=True, dsf=True, dtype=torch.bfloat16):
    x = gi.prefill_inputs(B, T, H, d, d, wid=wid, qkv_dtype=dtype, s0=s0, device=DEV)
    d_o = gi.draw_v((B, T, H, d), gi.seed_of(wid, 1, "v"), torch.float32, DEV)
    ds = gi.draw_state((B, H, d, d), gi.seed_of(wid, 1, "s0"), DEV) if dsf else None
    return x, d_o, ds


def run_case(B, T, H, rule, wid, s0=True, dsf=True, want_d_initial=True, dtype=torch.bfloat16, d=64, mutate=None):
    print(f"[case] backward B={B} T={T} H={H} d={d} rule={rule} s0={s0} dsf={dsf} {dtype}", flush=True)
    x, d_o, ds = grad_inputs(B, T, H, d, wid, s0, dsf, dtype)
    if mutate is not None:
        mutate(x)
    got = gdn.chunk_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_o, x["s0"], ds,
                             want_d_initial=want_d_initial, rule=rule)
    torch.cuda.synchronize()
    ref = oracle.backward(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["g"].cpu(), x["beta"].cpu(),
                          None if x["s0"] is None else x["s0"].cpu(), d_o.cpu(),
                          None if ds is None else ds.cpu(), rule=ORULE[rule])
    names = ("dq", "dk", "dv", "dg", "dbeta", "ds0")
    for name, t in zip(names, got):
        if t is None:
            continue
        if T == 0 and name != "ds0":
            continue
        tol = TOL["bf16"] if dtype == torch.bfloat16 else TOL["f32"]
        assert_parity(t.cpu().numpy(), ref[name], tol, f"{name} T={T} rule={rule} {dtype}")
    return got, ref


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
def test_backward_ragged(rule):
    run_case(2, 100, 3, rule, 210)


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
def test_backward_several_forward_pieces(rule):
    # 64 chunks of 32 tokens per head over 2 heads: the forward recompute runs in 8 pieces
    run_case(1, 2048, 2, rule, 211)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_forward_map_restart(d):
    """The forward recompute's map pass through its identity-slice drops and their restart: even
    32-token chunks decay hard (g = -1.1), odd ones have b = 1 and |k|^2 near 2.2 (a token map with
    an eigenvalue near -1.2), over 16 forward pieces per head, so every piece that drops a slice
    recomputes its map.  Every gradient against the oracle's adjoint."""
    def mutate(x):
        odd = ((torch.arange(x["g"].shape[1], device=DEV) // 32) % 2 == 1)[None, :, None]
        x["g"] = torch.where(odd, x["g"], torch.full_like(x["g"], -1.1))
        x["beta"] = torch.where(odd, torch.ones_like(x["beta"]), x["beta"])
        x["k"] = torch.where(odd[..., None], (x["k"].float() * 2.2 ** 0.5).to(torch.bfloat16), x["k"])
    run_case(1, 4096 + 19, 2, gdn.GDN_RULE_GATED_DELTA, 219, d=d, mutate=mutate)


def test_backward_without_state_or_final_gradient():
    run_case(2, 70, 2, gdn.GDN_RULE_GATED_DELTA, 212, s0=False, dsf=False)


def test_backward_without_initial_state_gradient():
    got, _ = run_case(1, 64, 2, gdn.GDN_RULE_GATED_DELTA, 213, want_d_initial=False)
    assert got[5] is None


@pytest.mark.parametrize("T", [0, 1, 31, 33])
def test_backward_short(T):
    run_case(2, T, 2, gdn.GDN_RULE_GATED_DELTA, 214 + T)


def test_backward_full_1b_8k():
    # the training shape B=4, H=32, T=8192, d=64 (the 1b_8k workload), every gradient element
    w = gi.WORKLOADS["1b_8k"]
    run_case(w.B, w.T, w.H, gdn.GDN_RULE_GATED_DELTA, w.wid, s0=True, dsf=True)


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
def test_backward_fp32_inputs(rule):
    # fp32 q/k/v: the forward recompute runs the fp32 chunk kernel; fp32 tolerance (1e-4 RMS)
    run_case(2, 100, 2, rule, 220, dtype=torch.float32)


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
def test_backward_two_level_scan(rule):
    # 150 chunks of 32 tokens on 2 heads: the reverse scan runs in pieces of 16 chunks (the last one
    # ragged: 6 chunks, its last chunk 4 tokens short)
    run_case(1, 150 * 32 - 4, 2, rule, 230)


def test_backward_two_level_scan_1b_64k_sampled():
    # the single 64K sequence (B=1 H=32 T=65536): pieces of 64 chunks.  The oracle runs on 2 of the
    # 32 heads (heads are independent: the same inputs restricted to those heads)
    B, T, H = 1, 65536, 32
    print(f"[case] backward 1b_64k T={T} H={H}", flush=True)
    x, d_o, ds = grad_inputs(B, T, H, 64, 3)
    got = gdn.chunk_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_o, x["s0"], ds)
    torch.cuda.synchronize()
    heads = [0, 21]
    sub = lambda t: t[:, :, heads].contiguous().cpu() if t.dim() >= 3 and t.shape[1] == T else t[:, heads].contiguous().cpu()
    ref = oracle.backward(sub(x["q"]), sub(x["k"]), sub(x["v"]), sub(x["g"]), sub(x["beta"]), sub(x["s0"]),
                          sub(d_o), sub(ds))
    for name, t in zip(("dq", "dk", "dv", "dg", "dbeta", "ds0"), got):
        assert_parity(sub(t).numpy(), ref[name], TOL["bf16"], f"{name} 1b_64k heads {heads}")


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_backward_d128_ragged(rule, dtype):
    # 128-wide heads: the gradient pass keeps its larger matrices in global scratch
    run_case(2, 100, 3, rule, 240, dtype=dtype, d=128)


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
def test_backward_d128_forward_pieces(rule):
    # 150 chunks on 2 heads: the forward recompute runs in pieces; one-level reverse scan (the last
    # chunk 4 tokens short)
    run_case(1, 150 * 32 - 4, 2, rule, 241, d=128)


def test_backward_d128_two_level_scan():
    # 1,100 chunks on 2 heads: the reverse scan runs in pieces of 64 chunks (the last piece 12
    # chunks, its last chunk 4 tokens short)
    run_case(1, 1100 * 32 - 4, 2, gdn.GDN_RULE_GATED_DELTA, 245, d=128)


def test_backward_d128_short_and_no_state():
    run_case(2, 33, 2, gdn.GDN_RULE_GATED_DELTA, 242, s0=False, dsf=False, d=128)
    run_case(1, 1, 2, gdn.GDN_RULE_GATED_DELTA, 243, d=128)


def test_backward_3b_shaped_8k_sampled_heads():
    # a 3B-shaped layer's 8K training call (B=1 H=24 T=8192 d=128); the oracle runs on 2 of the
    # 24 heads (heads are independent: the same inputs restricted to those heads)
    B, T, H, d = 1, 8192, 24, 128
    print(f"[case] backward 3b-shaped T={T} H={H} d={d}", flush=True)
    x, d_o, ds = grad_inputs(B, T, H, d, 244)
    got = gdn.chunk_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_o, x["s0"], ds)
    torch.cuda.synchronize()
    heads = [0, 17]
    sub = lambda t: t[:, :, heads].contiguous().cpu() if t.dim() >= 3 and t.shape[1] == T else t[:, heads].contiguous().cpu()
    ref = oracle.backward(sub(x["q"]), sub(x["k"]), sub(x["v"]), sub(x["g"]), sub(x["beta"]), sub(x["s0"]),
                          sub(d_o), sub(ds))
    for name, t in zip(("dq", "dk", "dv", "dg", "dbeta", "ds0"), got):
        assert_parity(sub(t).numpy(), ref[name], TOL["bf16"], f"{name} 3b-shaped heads {heads}")
