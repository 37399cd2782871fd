"""GPU parity of packed variable-length prefill with a state pool (MI355X only).

Each packed sequence must equal the fp64 oracle run on that sequence alone, from its pool slot's
state (or zeros), with its final state landing in its slot; slots no sequence uses stay bit for bit
as they were.  Covers empty, one-token and ragged sequences, sequences long enough to be split into
pieces, slot -1 (start from zeros, final state dropped) and both rules, on the MFMA chunk kernels
(bf16, 64- and 128-wide) and on the fp32 VALU kernel (fp32 q/k/v, and the 16-wide shapes)."""
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


def run_case(orc, lens, H, dk, dv, chunk, slots, init, pool_size, rule, rows=None, wid=80, dtype=torch.bfloat16,
             mutate=None):
    S, T = len(lens), int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tol = TOL["bf16"] if dtype == torch.bfloat16 else TOL["f32"]
    d = gi.prefill_inputs(1, T, H, dk, dv, wid=wid, qkv_dtype=dtype, device=DEV)
    d = {k: x[0] for k, x in d.items() if x is not None}
    if mutate is not None:
        mutate(d, cu)
    pool = gi.decode_state(pool_size, H, dk, dv, wid=wid + 1, device=DEV)
    pool0 = pool.clone()
    print(f"[case] varlen S={S} T={T} H={H} dk={dk} dv={dv} chunk={chunk} rule={rule} dtype={dtype}", flush=True)
    o = gdn.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, pool, slots=slots,
                                 has_initial=init, chunk=chunk, rule=rule)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    ref_o = np.full((T, H, dv), np.nan)
    p0 = pool0.cpu().numpy()
    expect_pool = p0.astype(np.float64).copy()
    for s in range(S):
        a, b = cu[s], cu[s + 1]
        sl = slots[s] if slots is not None else s
        start = p0[sl][None] if (sl >= 0 and (init is None or init[s])) else None
        if b > a:
            seq = {k: d[k][a:b][None] for k in ("q", "k", "v", "g", "beta")}
            ro, rs = orc.prefill(seq["q"], seq["k"], seq["v"], seq["g"], seq["beta"],
                                 None if start is None else torch.from_numpy(start), rows=rows, rule=ORULE[rule])
            ref_o[a:b] = ro[0]
            fin = rs[0]
        else:
            fin = start[0] if start is not None else np.zeros((H, dk, dv))
        if sl >= 0:
            expect_pool[sl] = fin
    assert_parity(o, ref_o, tol, "varlen outputs")
    used = sorted({(slots[s] if slots is not None else s) for s in range(S)} - {-1})
    got_pool = pool.cpu().numpy()
    assert_parity(got_pool[used], expect_pool[used], tol, "varlen final states")
    untouched = [i for i in range(pool_size) if i not in used]
    if untouched:
        assert np.array_equal(got_pool[untouched], p0[untouched]), "slots no sequence uses must not change"


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
@pytest.mark.parametrize("dk,dv,chunk", [(64, 64, 64), (128, 128, 64), (64, 128, 32)])
def test_varlen_matches_each_sequence(orc, rule, dk, dv, chunk):
    lens = [1000, 0, 63, 2500, 700, 1]
    slots = np.array([2, 5, -1, 0, 7, 4], dtype=np.int32)
    init = np.array([1, 0, 1, 1, 0, 1], dtype=np.int32)
    run_case(orc, lens, 3, dk, dv, chunk, slots, init, 8, rule)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
def test_varlen_map_drops_then_expanding_chunk(orc, dk, dv):
    """Packed sequences through the map pass's identity-slice drops and their restart: inside each
    sequence, even 32-token chunks decay hard (g = -1.1, the map falls far below 2^-32) and odd ones
    have b = 1 and |k|^2 near 2.2 (a token map with an eigenvalue near -1.2), so every piece that
    drops a slice restarts its map.  Each sequence against the oracle run on it alone."""
    def mutate(d, cu):
        pos = torch.zeros(d["g"].shape[0], dtype=torch.long, device=DEV)
        for s in range(len(cu) - 1):
            pos[cu[s]:cu[s + 1]] = torch.arange(cu[s + 1] - cu[s], device=DEV)
        odd = ((pos // 32) % 2 == 1)[:, None]
        d["g"] = torch.where(odd, d["g"], torch.full_like(d["g"], -1.1))
        d["beta"] = torch.where(odd, torch.ones_like(d["beta"]), d["beta"])
        d["k"] = torch.where(odd[..., None], (d["k"].float() * 2.2 ** 0.5).to(torch.bfloat16), d["k"])
    lens = [2500, 700, 3100, 40]
    slots = np.array([1, 3, 0, 2], dtype=np.int32)
    init = np.array([1, 1, 0, 1], dtype=np.int32)
    run_case(orc, lens, 2, dk, dv, 64, slots, init, 4, gdn.GDN_RULE_GATED_DELTA, mutate=mutate)


def test_varlen_default_slots_and_many_sequences(orc):
    """slots = None (sequence s uses slot s), 24 sequences of seeded random lengths, sampled rows."""
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(1, 1500, size=24)]
    run_case(orc, lens, 4, 64, 64, 64, None, None, 24, gdn.GDN_RULE_GATED_DELTA, rows=[0, 21, 38, 63])  # one row per 16-column slice


def test_varlen_equal_lengths_match_dense_prefill():
    """Two sequences of one length, packed, give what the dense [B, T] prefill gives."""
    T, H = 3000, 2
    d = gi.prefill_inputs(2, T, H, 64, 64, wid=85, qkv_dtype=torch.bfloat16, s0=True, device=DEV)
    o_dense, s_dense = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    pool = d["s0"].clone()
    packed = {k: d[k].reshape(2 * T, *d[k].shape[2:]).contiguous() for k in ("q", "k", "v", "g", "beta")}
    o = gdn.chunk_prefill_varlen(packed["q"], packed["k"], packed["v"], packed["g"], packed["beta"],
                                 [0, T, 2 * T], pool)
    torch.cuda.synchronize()
    ref = o_dense.reshape(2 * T, H, 64).cpu().numpy()
    assert_parity(o.cpu().numpy(), ref, 1e-3, "packed vs dense outputs")
    assert_parity(pool.cpu().numpy(), s_dense.cpu().numpy(), 1e-3, "packed vs dense final states")


@pytest.mark.parametrize("rule", [gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY])
@pytest.mark.parametrize("dtype,dk,dv,chunk", [(torch.float32, 64, 64, 64), (torch.float32, 128, 128, 32),
                                               (torch.float32, 16, 64, 16), (torch.bfloat16, 16, 16, 16),
                                               (torch.bfloat16, 64, 64, 16)])
def test_varlen_valu_kernel_matches_each_sequence(orc, rule, dtype, dk, dv, chunk):
    """fp32 q/k/v and the 16-wide shapes: the fp32 VALU kernel, one workgroup per sequence, head and
    16 value columns, to the fp32 bar (1e-4) for fp32 inputs."""
    lens = [700, 0, 45, 1, 1300, 33]
    slots = np.array([3, 1, -1, 0, 5, 2], dtype=np.int32)
    init = np.array([1, 0, 1, 0, 1, 1], dtype=np.int32)
    run_case(orc, lens, 3, dk, dv, chunk, slots, init, 6, rule, wid=88, dtype=dtype)


def test_varlen_valu_kernel_equals_dense_bitwise():
    """Two fp32 sequences of one length, packed, give bit for bit what the dense [B, T] prefill gives
    (the same VALU kernel on the same rows)."""
    T, H = 777, 3
    d = gi.prefill_inputs(2, T, H, 64, 64, wid=86, qkv_dtype=torch.float32, s0=True, device=DEV)
    o_dense, s_dense = gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    pool = d["s0"].clone()
    packed = {k: d[k].reshape(2 * T, *d[k].shape[2:]).contiguous() for k in ("q", "k", "v", "g", "beta")}
    o = gdn.chunk_prefill_varlen(packed["q"], packed["k"], packed["v"], packed["g"], packed["beta"],
                                 [0, T, 2 * T], pool)
    torch.cuda.synchronize()
    assert torch.equal(o, o_dense.reshape(2 * T, H, 64))
    assert torch.equal(pool, s_dense)
