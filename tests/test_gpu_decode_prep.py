"""GPU parity of gdn_prepare_decode_step, the decode step from the raw projections (MI355X only).

Over several consecutive tokens (convolution windows and states carried in place):
* against the fp64 oracles chained: oracle/prep.py's preparation of each token (window carried),
  then the decode oracle on its q, k, v.  The fused kernel keeps the prepared values in fp32 (no
  rounding to the storage type between the two steps), so outputs and final states are held to
  the fp32 bar (1e-4 of the RMS) for bf16 and fp32 inputs alike; the carried window is a copy of
  inputs and must match bit for bit;
* against the two separate launches (gdn_prepare, then gdn_decode_step_rule) for fp32 inputs,
  where neither path rounds: outputs and states to 1e-5 of the RMS (only the order of the norm's
  sum differs), windows bit for bit.  For bf16 inputs the separate path stores q, k, v as bf16;
  its own tests cover that rounding, and here only the windows are compared."""
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


def np64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def step_inputs(N, H, d, t, dtype, wid):
    x = gi.prep_inputs(N, 1, H, d, d, wid=wid, call=t, x_dtype=dtype, device=DEV)
    return {k: (v[:, 0] if k in ("xq", "xk", "xv", "a_raw", "b_raw") else v) for k, v in x.items()}


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("N,H,d", [(5, 3, 64), (256, 32, 64), (5, 3, 128), (256, 24, 128)])
def test_fused_step_matches_oracles_and_separate_launches(orc, rule, dtype, N, H, d):
    steps, wid = 3, 400 + N + d
    print(f"[case] prepare+decode fused N={N} H={H} d={d} {dtype} rule={rule}", flush=True)
    first = step_inputs(N, H, d, 0, dtype, wid)
    conv0 = first["conv_state"].clone()
    state0 = gi.decode_state(N, H, d, d, wid=wid, device=DEV)
    conv_f, state_f = conv0.clone(), state0.clone()   # fused
    conv_s, state_s = conv0.clone(), state0.clone()   # separate launches
    ref_conv, ref_state = np64(conv0), np64(state0).copy()
    orule = oracle.GATED_DELTA if rule == gdn.GDN_RULE_GATED_DELTA else oracle.GATED_DECAY
    HK = H * d
    outs_f, outs_s, refs = [], [], []
    for t in range(steps):
        x = step_inputs(N, H, d, t, dtype, wid)
        kw = dict(decay_rate=x["decay_rate"], gate_bias=x["gate_bias"])
        outs_f.append(gdn.prepare_decode_step(x["xq"], x["xk"], x["xv"], x["conv_weight"], x["a_raw"], x["b_raw"],
                                              conv_f, state_f, rule=rule, **kw))
        q, k, v, g, beta = gdn.prepare(x["xq"][:, None], x["xk"][:, None], x["xv"][:, None], x["conv_weight"],
                                       x["a_raw"][:, None], x["b_raw"][:, None], conv_state=conv_s,
                                       conv_state_out=conv_s, **kw)
        outs_s.append(gdn.decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], state_s, rule=rule))
        # the oracles, chained the same way
        w = np64(x["conv_weight"])
        r = oprep.prepare(x["xq"][:, None], x["xk"][:, None], x["xv"][:, None], w[:HK], w[HK:2 * HK], w[2 * HK:],
                          x["a_raw"][:, None], x["b_raw"][:, None], ref_conv, A=np64(x["decay_rate"]),
                          dt_bias=np64(x["gate_bias"]))
        ref_conv = r["conv_state"]
        refs.append(orc.decode_step(r["q"][:, 0], r["k"][:, 0], r["v"][:, 0], r["g"][:, 0], r["beta"][:, 0],
                                    ref_state, rule=orule))
    torch.cuda.synchronize()
    tol = TOL["f32"]
    o_f = np.stack([np64(o) for o in outs_f])
    assert_parity(o_f, np.stack(refs), tol, "fused outputs vs oracles")
    assert_parity(np64(state_f), ref_state, tol, "fused state vs oracles")
    assert np.array_equal(np64(conv_f), ref_conv), "convolution window vs oracle (copies of inputs)"
    if dtype == torch.float32:
        assert_parity(o_f, np.stack([np64(o) for o in outs_s]), 1e-5, "fused vs separate launches, outputs")
        assert_parity(np64(state_f), np64(state_s), 1e-5, "fused vs separate launches, state")
    assert torch.equal(conv_f, conv_s), "convolution window: fused vs separate launches"


def test_fused_step_without_rate_or_bias(orc):
    N, H, d = 7, 2, 64
    print("[case] prepare+decode fused, no rate / bias", flush=True)
    x = gi.prep_inputs(N, 1, H, d, d, wid=420, rate=False, device=DEV)
    x = {k: (v[:, 0] if k in ("xq", "xk", "xv", "a_raw", "b_raw") else v) for k, v in x.items()}
    conv, state = x["conv_state"].clone(), gi.decode_state(N, H, d, d, wid=420, device=DEV)
    ref_state = np64(state).copy()
    o = gdn.prepare_decode_step(x["xq"], x["xk"], x["xv"], x["conv_weight"], x["a_raw"], x["b_raw"], conv, state)
    torch.cuda.synchronize()
    w = np64(x["conv_weight"])
    r = oprep.prepare(x["xq"][:, None], x["xk"][:, None], x["xv"][:, None], w[:H * d], w[H * d:2 * H * d],
                      w[2 * H * d:], x["a_raw"][:, None], x["b_raw"][:, None], np64(x["conv_state"]))
    ref_o = orc.decode_step(r["q"][:, 0], r["k"][:, 0], r["v"][:, 0], r["g"][:, 0], r["beta"][:, 0], ref_state)
    assert_parity(np64(o), ref_o, TOL["f32"], "outputs")
    assert_parity(np64(state), ref_state, TOL["f32"], "state")


def test_fused_step_rejects_unsupported_heads():
    N, H = 2, 2
    x = gi.prep_inputs(N, 1, H, 16, 16, wid=421, device=DEV)
    x = {k: (v[:, 0] if k in ("xq", "xk", "xv", "a_raw", "b_raw") else v) for k, v in x.items()}
    state = torch.zeros((N, H, 16, 16), device=DEV)
    with pytest.raises(gdn.GdnError):
        gdn.prepare_decode_step(x["xq"], x["xk"], x["xv"], x["conv_weight"], x["a_raw"], x["b_raw"],
                                x["conv_state"], state)
