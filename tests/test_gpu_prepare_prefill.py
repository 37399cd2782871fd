"""GPU parity of gdn_prepare_chunk_prefill, the preparation done in the prefill's loads (MI355X only).

Reference: the fp64 preparation (oracle/prep.py) on the same raw inputs, its q, k, v rounded once to
bf16 (the call rounds its prepared q, k, v as gdn_prepare stores them), then the fp64 token-by-token
oracle; outputs and final states to the bf16 bar (2e-2 of the RMS).  The carried convolution window
must equal the oracle's exactly (it is a copy of raw inputs).  Every element on small shapes (short,
ragged, piece-split sequences, both rules, with and without carried windows and start states); the
64K layer shape on one value row of every 16-column slice."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import hybrid_linear_attention_gated_amd as gdn
import oracle
from oracle import prep as oprep
from parity import TOL, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ORULE = {gdn.GDN_RULE_GATED_DELTA: oracle.GATED_DELTA, gdn.GDN_RULE_GATED_DECAY: oracle.GATED_DECAY}


def inputs(B, T, H, d, wid, state=True, rate=True, s0=True):
    p = gi.prep_inputs(B, T, H, d, d, wid=wid, x_dtype=torch.bfloat16, state=state, rate=rate, device=DEV)
    p["s0"] = gi.draw_state((B, H, d, d), gi.seed_of(wid, 0, "s0"), DEV) if s0 else None
    return p


def reference(orc, p, rule, rows=None):
    B, T, H, dk = p["xq"].shape
    w = p["conv_weight"].cpu()
    r = oprep.prepare(p["xq"], p["xk"], p["xv"], w[:H * dk], w[H * dk:2 * H * dk], w[2 * H * dk:], p["a_raw"],
                      p["b_raw"], p["conv_state"], p["decay_rate"], p["gate_bias"])
    q, k, v = (torch.from_numpy(r[n]).to(torch.bfloat16) for n in ("q", "k", "v"))
    ro, rs = orc.prefill(q, k, v, r["g"], r["beta"], None if p["s0"] is None else p["s0"].cpu(), rows=rows,
                         rule=ORULE[rule])
    return ro, rs, r["conv_state"]


def run(p, rule, chunk=64, in_place=False):
    cout = p["conv_state"] if in_place else None
    if not in_place and p["conv_state"] is not None:
        cout = torch.empty_like(p["conv_state"])
    sf = p["s0"] if (in_place and p["s0"] is not None) else None
    o, sf = gdn.prepare_chunk_prefill(p["xq"], p["xk"], p["xv"], p["conv_weight"], p["a_raw"], p["b_raw"], p["s0"],
                                      decay_rate=p["decay_rate"], gate_bias=p["gate_bias"], conv_state=p["conv_state"],
                                      conv_state_out=cout, chunk=chunk, final_state=sf, rule=rule)
    torch.cuda.synchronize()
    return o, sf, cout


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
@pytest.mark.parametrize("B,T,H,d", [(2, 200, 3, 64), (1, 1, 2, 64), (1, 3, 2, 64), (2, 61, 3, 64), (1, 2500, 2, 64),
                                     (1, 700, 2, 128), (1, 2100, 1, 128)])
def test_prepared_prefill_matches_oracle(orc, rule, B, T, H, d):
    p = inputs(B, T, H, d, wid=140 + T % 97)
    print(f"[case] prepared prefill B={B} T={T} H={H} d={d} rule={rule}", flush=True)
    ref_o, ref_s, ref_w = reference(orc, p, rule)
    o, sf, cout = run(p, rule)
    assert_parity(o.cpu().numpy(), ref_o, TOL["bf16"], "prepared prefill outputs")
    assert_parity(sf.cpu().numpy(), ref_s, TOL["bf16"], "prepared prefill final state")
    assert np.array_equal(cout.cpu().double().numpy(), ref_w), "carried convolution window"


def test_prepared_prefill_without_window_rate_or_start_state(orc):
    p = inputs(2, 333, 2, 64, wid=151, state=False, rate=False, s0=False)
    print("[case] prepared prefill, zero window, no rate/bias, zero start state", flush=True)
    ref_o, ref_s, _ = reference(orc, p, gdn.GDN_RULE_GATED_DELTA)
    o, sf, _ = run(p, gdn.GDN_RULE_GATED_DELTA)
    assert_parity(o.cpu().numpy(), ref_o, TOL["bf16"], "outputs")
    assert_parity(sf.cpu().numpy(), ref_s, TOL["bf16"], "final state")


def test_prepared_prefill_equals_two_launches():
    """The same inputs through gdn_prepare + gdn_chunk_prefill.  The two paths sum each head's squared
    q and k norms in different orders, so a prepared value now and then rounds to the neighbouring bf16
    value; each path is held to the oracle on its own, and here to the same bf16 bar against the other."""
    p = inputs(1, 5000, 4, 64, wid=152)
    q, k, v, g, beta = gdn.prepare(p["xq"], p["xk"], p["xv"], p["conv_weight"], p["a_raw"], p["b_raw"],
                                   decay_rate=p["decay_rate"], gate_bias=p["gate_bias"], conv_state=p["conv_state"])
    o2, s2 = gdn.chunk_prefill(q, k, v, g, beta, p["s0"], chunk=64)
    o, sf, _ = run(p, gdn.GDN_RULE_GATED_DELTA)
    assert_parity(o.cpu().numpy(), o2.cpu().numpy(), TOL["bf16"], "fused vs two launches, outputs")
    assert_parity(sf.cpu().numpy(), s2.cpu().numpy(), TOL["bf16"], "fused vs two launches, state")


def test_prepared_prefill_in_place_chaining(orc):
    """Two chained calls (window and state updated in place): the carried window equals one call's, and
    both the chained outputs and the one-call outputs meet the bar against the oracle run once over the
    whole sequence (the split moves the chunk boundaries, so the two round differently)."""
    p = inputs(2, 3000, 3, 64, wid=153)
    o_one, s_one, w_one = run({**p, "conv_state": p["conv_state"].clone(), "s0": p["s0"].clone()},
                              gdn.GDN_RULE_GATED_DELTA)
    w, s = p["conv_state"].clone(), p["s0"].clone()
    outs = []
    for a, b in ((0, 1300), (1300, 3000)):
        part = {n: (x[:, a:b].contiguous() if n in ("xq", "xk", "xv", "a_raw", "b_raw") else x) for n, x in p.items()}
        part["conv_state"], part["s0"] = w, s
        o, _, _ = run(part, gdn.GDN_RULE_GATED_DELTA, in_place=True)
        outs.append(o)
    o_two = torch.cat(outs, dim=1)
    assert torch.equal(w, w_one), "carried window after two calls"
    ref_o, ref_s, ref_w = reference(orc, p, gdn.GDN_RULE_GATED_DELTA)
    assert np.array_equal(w.cpu().double().numpy(), ref_w), "carried window vs oracle"
    for what, o, st in (("two chained calls", o_two, s), ("one call", o_one, s_one)):
        assert_parity(o.cpu().numpy(), ref_o, TOL["bf16"], f"{what}, outputs")
        assert_parity(st.cpu().numpy(), ref_s, TOL["bf16"], f"{what}, state")


def test_prepared_prefill_64k_layer_shape(orc):
    """B=1 H=32 T=65536 d=64: one value row in every 16-column slice."""
    rows = [0, 21, 38, 63]
    p = inputs(1, 65536, 32, 64, wid=154)
    print("[case] prepared prefill B=1 H=32 T=65536", flush=True)
    o, sf, cout = run(p, gdn.GDN_RULE_GATED_DELTA)
    ref_o, ref_s, ref_w = reference(orc, p, gdn.GDN_RULE_GATED_DELTA, rows=rows)
    assert_parity(o.cpu().numpy()[..., rows], ref_o[..., rows], TOL["bf16"], f"64K outputs (rows {rows})")
    assert_parity(sf.cpu().numpy()[..., rows], ref_s[..., rows], TOL["bf16"], f"64K state (rows {rows})")
    assert np.array_equal(cout.cpu().double().numpy(), ref_w), "carried convolution window"
