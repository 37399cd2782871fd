"""GPU parity of the second rule, S_t = a_t S_{t-1} + b_t v_t k_t^T (no erase term), against the
fp64 oracle's evaluation of the same rule (MI355X only).  Same tolerances and coverage pattern as
the gated delta rule: every element on shapes spanning several chunks, pieces and ragged tails;
sampled value rows at the 64K workload's full size."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import hybrid_linear_attention_gated_amd as gdn
import oracle
from parity import TOL, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RULE = gdn.GDN_RULE_GATED_DECAY


def inputs(B, T, H, dk, dv, dtype, s0=True, gate="primary", wid=70, call=0):
    return gi.prefill_inputs(B, T, H, dk, dv, wid=wid, call=call, qkv_dtype=dtype, gate=gate, s0=s0,
                             device=DEV)


def check(orc, d, chunk, tol, what, rows=None):
    print(f"[case] decay rule {what} chunk={chunk}", flush=True)
    o, sf = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk=chunk, rule=RULE)
    torch.cuda.synchronize()
    ro, rs = orc.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], rows=rows, rule=oracle.GATED_DECAY)
    assert_parity(o.cpu().numpy(), ro, tol, what + " outputs")
    assert_parity(sf.cpu().numpy(), rs, tol, what + " final state")


@pytest.mark.parametrize("gate", ["primary", "literal"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128)])
@pytest.mark.parametrize("chunk", [32, 64])
def test_decay_bf16_mfma_path(orc, gate, dk, dv, chunk):
    d = inputs(2, 3 * chunk + 7, 3, dk, dv, torch.bfloat16, gate=gate)
    check(orc, d, chunk, TOL["bf16"], f"bf16 dk={dk} dv={dv} gate={gate}")


@pytest.mark.parametrize("dk,dv,chunk,T,s0", [(64, 64, 64, 2560, True), (64, 64, 64, 2547, False),
                                               (128, 128, 64, 2560, True), (64, 128, 32, 2600, True)])
def test_decay_sequence_pieces(orc, dk, dv, chunk, T, s0):
    d = inputs(1, T, 2, dk, dv, torch.bfloat16, s0=s0)
    check(orc, d, chunk, TOL["bf16"], f"pieces T={T} dk={dk} dv={dv}")


@pytest.mark.parametrize("dk,dv,chunk", [(16, 16, 16), (64, 64, 64), (128, 64, 32), (16, 64, 64)])
def test_decay_fp32_path(orc, dk, dv, chunk):
    d = inputs(2, 2 * chunk + 5, 2, dk, dv, torch.float32)
    check(orc, d, chunk, TOL["f32"], f"fp32 dk={dk} dv={dv}")


@pytest.mark.parametrize("T", [1, 63, 65])
def test_decay_short_and_ragged(orc, T):
    d = inputs(2, T, 2, 64, 64, torch.bfloat16)
    check(orc, d, 64, TOL["bf16"], f"T={T}")


def test_decay_differs_from_the_delta_rule():
    """The two rules give different results on the same inputs (the rule argument is honoured)."""
    d = inputs(1, 200, 2, 64, 64, torch.bfloat16, gate="primary")
    o1, _ = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], rule=RULE)
    o2, _ = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() > 1e-2 * o2.pow(2).mean().sqrt().item()


def test_decay_decode_steps_match_oracle_and_prefill(orc):
    N, H, dk, dv, steps = 8, 4, 64, 64, 6
    state = gi.decode_state(N, H, dk, dv, device=DEV)
    ref_state = state.cpu().double().numpy().copy()
    start = state.clone()
    outs, ref_outs, ins = [], [], []
    for s in range(steps):
        d = gi.decode_inputs(N, H, dk, dv, s, device=DEV)
        ins.append(d)
        outs.append(gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, rule=RULE).cpu().numpy())
        ref_outs.append(orc.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], ref_state,
                                        rule=oracle.GATED_DECAY))
    torch.cuda.synchronize()
    assert_parity(np.stack(outs), np.stack(ref_outs), TOL["bf16"], "decay decode outputs")
    assert_parity(state.cpu().numpy(), ref_state, TOL["bf16"], "decay decode state")
    # the same tokens through prefill (sequence n = batch n) from the same start state
    cat = {k: torch.stack([x[k] for x in ins], dim=1) for k in ("q", "k", "v", "g", "beta")}
    o, sf = gdn.chunk_prefill(cat["q"], cat["k"], cat["v"], cat["g"], cat["beta"], start, rule=RULE)
    torch.cuda.synchronize()
    assert_parity(o.cpu().numpy(), np.stack(ref_outs, axis=1), TOL["bf16"], "decay prefill of the decode tokens")


def test_decay_workload_1b_64k_sampled_rows(orc):
    """The 64K workload's shape (B=1, H=32, T=65536, d=64, chunk 64, start state carried in) under
    the decay rule, compared on sampled value rows."""
    d = gi.workload_inputs("1b_64k", device=DEV)
    rows = [0, 17, 38, 63]
    check(orc, d, 64, TOL["bf16"], "1b_64k shape", rows=rows)
