"""Packed-sequence calls under HIP graph capture (MI355X only).

gdn_chunk_prefill_varlen and gdn_prepare_varlen copy a table built from host
arrays into the workspace.  A graph recorded from that copy would keep a pointer
to host memory that is freed when the call returns, so both calls refuse a
capturing stream with GDN_ERR_CAPTURE before queuing anything: the capture
records nothing of theirs, and replaying it leaves their outputs and pools as
they were.  The same calls made eagerly afterwards work as usual."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import hybrid_linear_attention_gated_amd as gdn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CAPTURE = 8


def test_packed_calls_refuse_capture_without_side_effects():
    H, d = 2, 64
    lens = [300, 1, 77]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    print(f"[case] capture: packed prefill and pooled preparation, T={T} H={H}", flush=True)
    x = gi.prefill_inputs(1, T, H, d, d, wid=91, qkv_dtype=torch.bfloat16, device=DEV)
    x = {k: t[0] for k, t in x.items() if t is not None}
    pool = gi.decode_state(3, H, d, d, wid=92, device=DEV)
    pool0 = pool.clone()
    o = torch.full((T, H, d), 7.0, device=DEV)
    ws = torch.full((gdn.varlen_workspace_bytes(cu, H, d, d, 64, gdn.GDN_BF16),), 3, dtype=torch.uint8,
                    device=DEV)

    p = gi.prep_inputs(1, T, H, d, d, wid=93, x_dtype=torch.bfloat16, state=False, device=DEV)
    C = H * (3 * d)
    conv_pool = torch.randn(3, C, 3, device=DEV)
    conv_pool0 = conv_pool.clone()
    outs = (torch.full((T, H, d), 1.5, device=DEV, dtype=torch.bfloat16),
            torch.full((T, H, d), 1.5, device=DEV, dtype=torch.bfloat16),
            torch.full((T, H, d), 1.5, device=DEV, dtype=torch.bfloat16),
            torch.full((T, H), 2.5, device=DEV), torch.full((T, H), 2.5, device=DEV))
    ws_prep = torch.full((gdn.gdn_prepare_varlen_workspace_size(len(lens)),), 4, dtype=torch.uint8, device=DEV)

    marker = torch.zeros(4, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    codes = []
    with torch.cuda.graph(graph):
        try:
            gdn.chunk_prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, pool, out=o, workspace=ws)
        except gdn.GdnError as e:
            codes.append(e.status)
        try:
            gdn.prepare_varlen(p["xq"][0], p["xk"][0], p["xv"][0], p["conv_weight"], p["a_raw"][0], p["b_raw"][0],
                               cu, conv_pool, decay_rate=p["decay_rate"], gate_bias=p["gate_bias"], outs=outs, workspace=ws_prep)
        except gdn.GdnError as e:
            codes.append(e.status)
        marker.add_(1.0)  # something the graph does record
    assert codes == [CAPTURE, CAPTURE]
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
    assert torch.all(marker == 3.0)
    assert torch.all(o == 7.0) and torch.equal(pool, pool0) and torch.all(ws == 3)
    assert all(torch.all(t == v) for t, v in zip(outs, (1.5, 1.5, 1.5, 2.5, 2.5)))
    assert torch.equal(conv_pool, conv_pool0) and torch.all(ws_prep == 4)

    # eagerly, on the same buffers, both calls run
    gdn.chunk_prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, pool, out=o, workspace=ws)
    gdn.prepare_varlen(p["xq"][0], p["xk"][0], p["xv"][0], p["conv_weight"], p["a_raw"][0], p["b_raw"][0], cu,
                       conv_pool, decay_rate=p["decay_rate"], gate_bias=p["gate_bias"], outs=outs, workspace=ws_prep)
    torch.cuda.synchronize()
    assert not torch.all(o == 7.0) and torch.isfinite(o).all()
    assert not torch.equal(pool, pool0) and not torch.equal(conv_pool, conv_pool0)
