"""gdn_chunk_prefill_noalloc, the allocation-free prefill (MI355X only).

Called through the C ABI, it must give what gdn_chunk_prefill_rule gives with a
workspace of the caller's: the same kernels run on the same piece plan, so the
outputs and final states agree bit for bit (and so within the bf16 bar of the
oracle parity tests).  For 128-wide heads under the gated delta rule the call
with a workspace keeps every chunk's T diag(b) fragments there and its second
pass reads them, where this call forms them again: the same arithmetic, so
still bit for bit.  Two calls in a row share the one static scratch array;
the second is smaller than the first, so it runs over the first call's leftover
maps and start states."""
import pytest
import torch

import gdn_inputs as gi
import hybrid_linear_attention_gated_amd as gdn
from parity import TOL, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def call_noalloc(d, B, T, H, dk, dv, rule):
    o = torch.full((B, T, H, dv), 3.0, device=DEV)
    sf = torch.full((B, H, dk, dv), 4.0, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    st = gdn.gdn_chunk_prefill_noalloc(rule, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                                       d["g"].data_ptr(), d["beta"].data_ptr(), d["s0"].data_ptr(), o.data_ptr(),
                                       sf.data_ptr(), B, T, H, dk, dv, 64, gdn.GDN_BF16, stream)
    assert st == 0, gdn.gdn_status_string(st)
    return o, sf


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
def test_noalloc_matches_workspace_call_twice(rule):
    cases = [(1, 65536, 32, 64, 64), (2, 5000, 3, 128, 128), (1, 3001, 5, 64, 64)]  # later calls smaller
    for i, (B, T, H, dk, dv) in enumerate(cases):
        print(f"[case] noalloc call {i}: B={B} T={T} H={H} dk={dk} dv={dv} rule={rule}", flush=True)
        need = gdn.workspace_bytes(B, T, H, dk, dv, 64, gdn.GDN_BF16)
        assert 0 < need <= 64 << 20
        d = gi.prefill_inputs(B, T, H, dk, dv, wid=120 + i, qkv_dtype=torch.bfloat16, s0=True, device=DEV)
        o_ref, s_ref = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk=64, rule=rule)
        o, sf = call_noalloc(d, B, T, H, dk, dv, rule)
        torch.cuda.synchronize()
        e_o = rel_err(o.cpu().numpy(), o_ref.cpu().numpy())
        e_s = rel_err(sf.cpu().numpy(), s_ref.cpu().numpy())
        print(f"[parity] noalloc vs workspace call: outputs {e_o:.1e}, state {e_s:.1e}", flush=True)
        assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]
        assert torch.equal(o, o_ref) and torch.equal(sf, s_ref)


def test_noalloc_in_place_and_short_call():
    """final_state aliasing initial_state (chained calls), and a call that needs no scratch."""
    B, T, H, d = 1, 9000, 4, 64
    x = gi.prefill_inputs(B, T, H, d, d, wid=131, qkv_dtype=torch.bfloat16, s0=True, device=DEV)
    o_ref, s_ref = gdn.chunk_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], chunk=64)
    st = x["s0"].clone()
    o = torch.empty_like(o_ref)
    code = gdn.gdn_chunk_prefill_noalloc(gdn.GDN_RULE_GATED_DELTA, x["q"].data_ptr(), x["k"].data_ptr(),
                                         x["v"].data_ptr(), x["g"].data_ptr(), x["beta"].data_ptr(), st.data_ptr(),
                                         o.data_ptr(), st.data_ptr(), B, T, H, d, d, 64, gdn.GDN_BF16,
                                         torch.cuda.current_stream().cuda_stream)
    assert code == 0
    y = gi.prefill_inputs(1, 100, 2, d, d, wid=132, qkv_dtype=torch.bfloat16, s0=True, device=DEV)
    assert gdn.workspace_bytes(1, 100, 2, d, d, 64, gdn.GDN_BF16) == 0
    oy_ref, sy_ref = gdn.chunk_prefill(y["q"], y["k"], y["v"], y["g"], y["beta"], y["s0"], chunk=64)
    oy, sy = call_noalloc(y, 1, 100, 2, d, d, gdn.GDN_RULE_GATED_DELTA)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(st, s_ref)
    assert torch.equal(oy, oy_ref) and torch.equal(sy, sy_ref)


@pytest.mark.parametrize("dk", [64, 128])
def test_noalloc_map_restart_matches_workspace_call(dk):
    """Inputs that make the map pass drop identity slices and then restart a piece's map (even 32-token
    chunks decay hard, odd ones have b = 1 and |k|^2 near 2.2): the allocation-free call still equals
    the call with a workspace bit for bit."""
    B, T, H = 1, 4096 + 19, 2
    d = gi.prefill_inputs(B, T, H, dk, dk, wid=133, qkv_dtype=torch.bfloat16, s0=True, device=DEV)
    odd = ((torch.arange(T, device=DEV) // 32) % 2 == 1)[None, :, None]
    d["g"] = torch.where(odd, d["g"], torch.full_like(d["g"], -1.1))
    d["beta"] = torch.where(odd, torch.ones_like(d["beta"]), d["beta"])
    d["k"] = torch.where(odd[..., None], (d["k"].float() * 2.2 ** 0.5).to(torch.bfloat16), d["k"])
    print(f"[case] noalloc restart: B={B} T={T} H={H} d={dk}", flush=True)
    o_ref, s_ref = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk=64)
    o, sf = call_noalloc(d, B, T, H, dk, dk, gdn.GDN_RULE_GATED_DELTA)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(sf, s_ref)
