"""GPU parity of gdn_decode_step against the fp64 oracle (MI355X only)."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import hybrid_linear_attention_gated_amd as gdn
from parity import TOL, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_chain(orc, N, H, dk, dv, steps, dtype, gate="primary"):
    state = gi.decode_state(N, H, dk, dv, device=DEV)
    ref_state = state.detach().cpu().double().numpy().copy()
    outs, refs = [], []
    for step in range(steps):
        d = gi.decode_inputs(N, H, dk, dv, step, qkv_dtype=dtype, gate=gate, device=DEV)
        o = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
        outs.append(o.cpu().numpy())
        refs.append(orc.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], ref_state))
    torch.cuda.synchronize()
    return np.stack(outs), np.stack(refs), state.cpu().numpy(), ref_state


@pytest.mark.parametrize("gate", ["primary", "literal"])
def test_decode_256_sequences_16_steps(orc, gate):
    """256 sequences, H=32, d=64, 16 consecutive steps, bf16 q/k/v, fp32 state."""
    print(f"[case] decode N=256 H=32 d=64 steps=16 gate={gate}", flush=True)
    o, ro, s, rs = run_chain(orc, 256, 32, 64, 64, 16, torch.bfloat16, gate)
    assert_parity(o, ro, TOL["bf16"], "decode outputs (16 steps)")
    assert_parity(s, rs, TOL["bf16"], "decode state after 16 steps")
    # the arithmetic is fp32 throughout: far tighter than the bf16 bar
    assert_parity(o, ro, 1e-5, "decode outputs, fp32-arithmetic bound")


@pytest.mark.parametrize("dk", [16, 64, 128])
@pytest.mark.parametrize("dv", [16, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_shapes(orc, dk, dv, dtype):
    print(f"[case] decode N=5 H=3 dk={dk} dv={dv} {dtype}", flush=True)
    o, ro, s, rs = run_chain(orc, 5, 3, dk, dv, 3, dtype)
    assert_parity(o, ro, TOL["f32"], "decode outputs")
    assert_parity(s, rs, TOL["f32"], "decode state")


def test_decode_is_deterministic_and_in_place():
    N, H, d = 64, 8, 64
    s0 = gi.decode_state(N, H, d, d, device=DEV)
    inp = gi.decode_inputs(N, H, d, d, 0, device=DEV)
    s1, s2 = s0.clone(), s0.clone()
    ptr = s1.data_ptr()
    o1 = gdn.decode_step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s1)
    o2 = gdn.decode_step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s2)
    torch.cuda.synchronize()
    assert s1.data_ptr() == ptr
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert not torch.equal(s1, s0)


def test_decode_graph_replays_match_eager():
    """Steps captured in a HIP graph (as a serving loop issues them) give, on every replay, the
    same outputs and state as the eager calls; the state is reset and read back between replays
    by ordinary eager work."""
    N, H, d, steps = 32, 8, 64, 4
    print(f"[case] decode graph N={N} H={H} d={d} steps={steps}", flush=True)
    s0 = gi.decode_state(N, H, d, d, device=DEV)
    inp = [gi.decode_inputs(N, H, d, d, t, device=DEV) for t in range(steps)]
    state = s0.clone()
    outs = [torch.empty((N, H, d), device=DEV, dtype=torch.float32) for _ in range(steps)]
    for x, o in zip(inp, outs):
        gdn.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, out=o)
    torch.cuda.synchronize()
    ref_o, ref_s = [o.clone() for o in outs], state.clone()

    graph = torch.cuda.CUDAGraph()
    state.copy_(s0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for x, o in zip(inp, outs):
            gdn.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, out=o)
    for rep in range(3):
        state.copy_(s0)
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, ref_s), f"replay {rep}: state"
        for t, (o, r) in enumerate(zip(outs, ref_o)):
            assert torch.equal(o, r), f"replay {rep}: step {t} outputs"


def test_decode_guard_regions_untouched():
    """Canary words around the state and output stay intact."""
    N, H, d = 33, 5, 64
    pad = 1024
    inp = gi.decode_inputs(N, H, d, d, 0, device=DEV)
    sbuf = torch.full((pad + N * H * d * d + pad,), 7.25, device=DEV)
    obuf = torch.full((pad + N * H * d + pad,), -3.5, device=DEV)
    state = sbuf[pad:pad + N * H * d * d].view(N, H, d, d)
    state.copy_(gi.decode_state(N, H, d, d, device=DEV))
    out = obuf[pad:pad + N * H * d].view(N, H, d)
    gdn.decode_step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], state, out=out)
    torch.cuda.synchronize()
    for buf, val in ((sbuf, 7.25), (obuf, -3.5)):
        assert torch.all(buf[:pad] == val) and torch.all(buf[-pad:] == val)


def test_decode_error_leaves_buffers_untouched():
    N, H, d = 4, 2, 64
    inp = gi.decode_inputs(N, H, d, d, 0, device=DEV)
    state = gi.decode_state(N, H, d, d, device=DEV)
    before = state.clone()
    st = gdn.gdn_decode_step(inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                             inp["g"].data_ptr(), inp["beta"].data_ptr(), state.data_ptr(),
                             inp["q"].data_ptr(), N, H, d, d, gdn.GDN_BF16, None)
    torch.cuda.synchronize()
    assert st == 5  # o aliases q
    assert torch.equal(state, before)


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
@pytest.mark.parametrize("d_head", [64, 128])
def test_decode_with_state_slots(orc, rule, d_head):
    """States in a pool of 10 slots; six sequences use slots 3, 7, 0, 9 and two padding entries
    (-1 and 12, out of range): valid slots follow the oracle, padding outputs are zero, every
    other slot is left bit for bit as it was (64-wide states take two wavefronts each, 128-wide
    eight, every one of which handles the padding entries on its own)."""
    import oracle
    print(f"[case] decode slots d={d_head} rule={rule}", flush=True)
    N, H, dk, dv, P = 6, 4, d_head, d_head, 10
    slots = torch.tensor([3, 7, -1, 0, 12, 9], dtype=torch.int32, device=DEV)
    pool = gi.decode_state(P, H, dk, dv, device=DEV)
    pool0 = pool.clone()
    ref = pool.cpu().double().numpy().copy()
    orule = oracle.GATED_DELTA if rule == gdn.GDN_RULE_GATED_DELTA else oracle.GATED_DECAY
    outs, refs = [], []
    for s in range(3):
        d = gi.decode_inputs(N, H, dk, dv, s, device=DEV)
        outs.append(gdn.decode_step_slots(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, slots,
                                          rule=rule).cpu().numpy())
        valid = [n for n, sl in enumerate(slots.tolist()) if 0 <= sl < P]
        sel = [slots[n].item() for n in valid]
        st = np.ascontiguousarray(ref[sel])
        ro = orc.decode_step(d["q"][valid], d["k"][valid], d["v"][valid], d["g"][valid], d["beta"][valid],
                             st, rule=orule)
        ref[sel] = st
        full = np.zeros((N, H, dv))
        full[valid] = ro
        refs.append(full)
    torch.cuda.synchronize()
    got = np.stack(outs)
    assert np.all(got[:, [2, 4]] == 0.0), "padding entries must output zeros"
    assert_parity(got[:, [0, 1, 3, 5]], np.stack(refs)[:, [0, 1, 3, 5]], TOL["bf16"], "slot decode outputs")
    used = [3, 7, 0, 9]
    assert_parity(pool.cpu().numpy()[used], ref[used], TOL["bf16"], "slot decode states")
    untouched = [i for i in range(P) if i not in used]
    assert torch.equal(pool[untouched], pool0[untouched]), "unused slots must not change"
