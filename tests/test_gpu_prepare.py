"""GPU parity of the input preparation ahead of the mixer (MI355X only).

The HIP kernel's q, k, v, g, beta and carried convolution state are compared element by element
with the fp64 reference in oracle/prep.py on the same seeded inputs.

Bound, per element, from the arithmetic: the kernel evaluates in fp32 (the convolution as four
fused multiply-adds, SiLU with the hardware exp and reciprocal, the norm with the hardware
reciprocal square root), which keeps it within a few 1e-7 of the exact value in units of the
tensor's RMS (a convolution of four O(1) terms, a Lipschitz-1 activation, a normalisation).
fp32 outputs: |err| <= 1e-5 |ref| + 4e-6 RMS.  bf16 outputs are that value rounded once to
nearest, whose relative error is at most the unit roundoff of an 8-bit significand, 2^-8:
|err| <= 2^-8 |ref| + 4.1e-6 RMS.  The gates (fp32, library exp/log1p) and the carried
state (copies of stored inputs) are held to 1e-5 |ref| + 1e-7 RMS and to exact equality."""
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
    return None if t is None else t.detach().cpu().to(torch.float64).numpy()


def assert_elementwise(got, ref, rel, rms_floor, what):
    got, ref = np64(got) if isinstance(got, torch.Tensor) else got, np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = rel * np.abs(ref) + rms_floor * rms
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if ref.size else 0.0
    print(f"[parity] {what}: max err/bound = {worst:.3f} (rel {rel:.1e}, floor {rms_floor:.1e} RMS)", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert worst <= 1.0, f"{what}: max err/bound = {worst:.3f}"


def bounds(dtype):
    return (2.0 ** -8, 4.1e-6) if dtype == torch.bfloat16 else (1e-5, 4e-6)


def check(outs, d, ref, dtype, what, state_out=None):
    q, k, v, g, beta = outs
    rel, floor = bounds(dtype)
    for name, got in (("q", q), ("k", k), ("v", v)):
        assert_elementwise(got, ref[name], rel, floor, f"{what} {name}")
    assert_elementwise(g, ref["g"], 1e-5, 1e-7, f"{what} g")
    assert_elementwise(beta, ref["beta"], 1e-5, 1e-7, f"{what} beta")
    if state_out is not None:
        assert np.array_equal(np64(state_out), ref["conv_state"]), f"{what}: carried state"


DEFAULT = object()


def reference(d, conv_state=DEFAULT):
    H = d["xq"].shape[2]
    dk, dv = d["xq"].shape[-1], d["xv"].shape[-1]
    w = np64(d["conv_weight"])
    st = d["conv_state"] if conv_state is DEFAULT else conv_state
    return oprep.prepare(d["xq"], d["xk"], d["xv"], w[:H * dk], w[H * dk:2 * H * dk], w[2 * H * dk:],
                         d["a_raw"], d["b_raw"], None if st is None else np64(st),
                         A=np64(d["decay_rate"]), dt_bias=np64(d["gate_bias"]))


def run(d, state_out=None, conv_state=DEFAULT):
    st = d["conv_state"] if conv_state is DEFAULT else conv_state
    outs = gdn.prepare(d["xq"], d["xk"], d["xv"], d["conv_weight"], d["a_raw"], d["b_raw"],
                       decay_rate=d["decay_rate"], gate_bias=d["gate_bias"], conv_state=st,
                       conv_state_out=state_out)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (16, 16), (128, 128), (64, 128), (16, 128)])
def test_prepare_matches_oracle(dk, dv, dtype):
    B, T, H = 2, 150, 3  # 3 token tiles (64 + 64 + 22); channel space not a multiple of a workgroup
    print(f"[case] prepare B={B} T={T} H={H} dk={dk} dv={dv} {dtype}", flush=True)
    d = gi.prep_inputs(B, T, H, dk, dv, wid=90 + dk + dv, x_dtype=dtype, device=DEV)
    st_out = torch.empty_like(d["conv_state"])
    outs = run(d, state_out=st_out)
    check(outs, d, reference(d), dtype, f"dk={dk} dv={dv}", state_out=st_out)


def test_prepare_without_state_rate_or_bias():
    print("[case] prepare no state / rate / bias", flush=True)
    d = gi.prep_inputs(1, 70, 2, 64, 64, wid=120, state=False, rate=False, device=DEV)
    outs = run(d)
    check(outs, d, reference(d), torch.bfloat16, "no state")


@pytest.mark.parametrize("T", [1, 2, 3, 64, 65])
def test_short_calls_update_the_state_in_place(T):
    print(f"[case] prepare in place T={T}", flush=True)
    d = gi.prep_inputs(3, T, 2, 64, 64, wid=130 + T, device=DEV)
    ref = reference(d)
    state = d["conv_state"].clone()
    outs = run(d, state_out=state, conv_state=state)
    check(outs, d, ref, torch.bfloat16, f"T={T} in place", state_out=state)


def test_long_call_updates_the_state_in_place():
    # several tiles: the new state is written by a second launch after the old one is read
    print("[case] prepare in place T=200", flush=True)
    d = gi.prep_inputs(2, 200, 2, 128, 64, wid=140, device=DEV)
    ref = reference(d)
    state = d["conv_state"].clone()
    outs = run(d, state_out=state, conv_state=state)
    check(outs, d, ref, torch.bfloat16, "T=200 in place", state_out=state)


def test_zero_tokens_carry_the_state():
    print("[case] prepare T=0", flush=True)
    d = gi.prep_inputs(2, 0, 2, 64, 64, wid=150, device=DEV)
    out = torch.full_like(d["conv_state"], 7.0)
    run(d, state_out=out)
    assert torch.equal(out, d["conv_state"])
    zero_out = torch.full_like(d["conv_state"], 7.0)
    run(d, state_out=zero_out, conv_state=None)
    assert torch.count_nonzero(zero_out).item() == 0


def test_split_calls_equal_one_call_bit_for_bit():
    print("[case] prepare chaining 37 + 163", flush=True)
    d = gi.prep_inputs(2, 200, 3, 64, 64, wid=160, device=DEV)
    whole = run(d, state_out=torch.empty_like(d["conv_state"]))
    cut = 37
    first = {k: (x[:, :cut].contiguous() if k in ("xq", "xk", "xv", "a_raw", "b_raw") else x) for k, x in d.items()}
    rest = {k: (x[:, cut:].contiguous() if k in ("xq", "xk", "xv", "a_raw", "b_raw") else x) for k, x in d.items()}
    state = d["conv_state"].clone()
    a = run(first, state_out=state, conv_state=state)
    b = run(rest, state_out=state, conv_state=state)
    for i, name in enumerate(("q", "k", "v", "g", "beta")):
        assert torch.equal(torch.cat([a[i], b[i]], dim=1), whole[i]), name
    check(tuple(torch.cat([a[i], b[i]], dim=1) for i in range(5)), d, reference(d), torch.bfloat16, "chained")


def test_decode_shape_in_place():
    # the serving decode step: one token for each of 256 sequences, state carried in place
    print("[case] prepare decode N=256 H=32", flush=True)
    d = gi.prep_inputs(256, 1, 32, 64, 64, wid=170, device=DEV)
    ref = reference(d)
    state = d["conv_state"].clone()
    outs = run(d, state_out=state, conv_state=state)
    check(outs, d, ref, torch.bfloat16, "decode", state_out=state)


def test_full_size_sampled_rows():
    # B=1, T=65536, H=32, d=64 bf16 (the 64K prefill's shape): sampled tokens against the oracle on
    # each token's own 4-token window (the convolution looks back 3 tokens), properties everywhere
    B, T, H, dk, dv = 1, 65536, 32, 64, 64
    print(f"[case] prepare full size T={T} H={H}", flush=True)
    d = gi.prep_inputs(B, T, H, dk, dv, wid=180, device=DEV)
    outs = run(d, state_out=torch.empty_like(d["conv_state"]))
    q, k, v, g, beta = outs
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 1, 2, 3, 62, 63, 64, 65, 127, 128, 4095, 4096, T - 2, T - 1] +
                      rng.integers(0, T, 48).tolist()))
    cpu = {kk: (x.cpu() if isinstance(x, torch.Tensor) else x) for kk, x in d.items()}
    rel, floor = bounds(torch.bfloat16)
    for t in rows:
        lo = max(0, t - 3)
        win = {kk: (x[:, lo:t + 1] if kk in ("xq", "xk", "xv", "a_raw", "b_raw") else x) for kk, x in cpu.items()}
        ref = reference(win, conv_state=cpu["conv_state"] if t < 3 else None)
        for name, got in (("q", q), ("k", k), ("v", v)):
            r = ref[name][:, -1]
            gg = np64(got[:, t])
            # RMS of the full tensor is ~1/sqrt(d) for q, k and ~0.6 for v; use the window's own RMS
            assert np.all(np.abs(gg - r) <= rel * np.abs(r) + floor * np.sqrt(np.mean(r * r))), (name, t)
        assert np.all(np.abs(np64(g[:, t]) - ref["g"][:, -1]) <= 1e-5 * np.abs(ref["g"][:, -1]) + 1e-12), ("g", t)
        assert np.all(np.abs(np64(beta[:, t]) - ref["beta"][:, -1]) <= 1e-5 * ref["beta"][:, -1]), ("beta", t)
    # properties over every token: unit q/k rows (up to eps and bf16 rounding), gates in range
    for name, x in (("q", q), ("k", k)):
        n2 = x.float().pow(2).sum(-1)
        assert float((n2 - 1).abs().max()) < 2e-2, name
    assert float(g.max()) <= 0.0 and float(beta.min()) > 0.0 and float(beta.max()) < 1.0
    assert torch.isfinite(v.float()).all()


def test_prepared_inputs_drive_the_mixer():
    # end to end: preparation then the chunked prefill, against the oracle's preparation (rounded to
    # bf16 as stored) then the oracle's rule
    B, T, H, dk, dv = 1, 300, 4, 64, 64
    print(f"[case] prepare -> chunk_prefill T={T}", flush=True)
    d = gi.prep_inputs(B, T, H, dk, dv, wid=190, device=DEV)
    q, k, v, g, beta = run(d)
    o, _ = gdn.chunk_prefill(q, k, v, g, beta, None, 64)
    torch.cuda.synchronize()
    ref = reference(d)
    as_bf16 = {n: torch.from_numpy(ref[n]).to(torch.bfloat16) for n in ("q", "k", "v")}
    ro, _ = oracle.prefill(as_bf16["q"], as_bf16["k"], as_bf16["v"], torch.from_numpy(ref["g"]).float(),
                           torch.from_numpy(ref["beta"]).float(), None)
    assert_parity(o.cpu().numpy(), ro, TOL["bf16"], "prepare -> prefill outputs")


# ---- packed sequences with a pool of convolution states -------------------------------------------------

def varlen_case(lens, H, dk, dv, pool_size, slots, init, dtype=torch.bfloat16, wid=300):
    S, T = len(lens), int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = gi.prep_inputs(1, T, H, dk, dv, wid=wid, x_dtype=dtype, state=False, device=DEV)
    x = {kk: (t[0] if kk in ("xq", "xk", "xv", "a_raw", "b_raw") else t) for kk, t in d.items()}
    C = H * (2 * dk + dv)
    pool = gi._normal((pool_size, C, 3), gi.seed_of(wid, 7, "conv_state"), DEV).to(dtype).float()
    pool0 = pool.clone()
    print(f"[case] prepare_varlen S={S} T={T} H={H} dk={dk} dv={dv} pool={pool_size} {dtype}", flush=True)
    q, k, v, g, beta = gdn.prepare_varlen(x["xq"], x["xk"], x["xv"], x["conv_weight"], x["a_raw"], x["b_raw"], cu,
                                          pool, slots=slots, has_initial=init, decay_rate=x["decay_rate"],
                                          gate_bias=x["gate_bias"])
    torch.cuda.synchronize()
    rel, floor = bounds(dtype)
    p0 = np64(pool0)
    expect = p0.copy()
    used = []
    for s in range(S):
        a, b = cu[s], cu[s + 1]
        sl = slots[s] if slots is not None else s
        start = p0[sl][None] if (sl >= 0 and (init is None or init[s])) else None
        seq = {kk: (x[kk][a:b][None] if kk in ("xq", "xk", "xv", "a_raw", "b_raw") else t) for kk, t in d.items()}
        ref = reference({kk: (t.cpu() if isinstance(t, torch.Tensor) else t) for kk, t in seq.items()},
                        conv_state=None if start is None else torch.from_numpy(start))
        if b > a:
            for name, got in (("q", q), ("k", k), ("v", v)):
                assert_elementwise(got[a:b][None], ref[name], rel, floor, f"seq {s} {name}")
            assert_elementwise(g[a:b][None], ref["g"], 1e-5, 1e-7, f"seq {s} g")
            assert_elementwise(beta[a:b][None], ref["beta"], 1e-5, 1e-7, f"seq {s} beta")
        if sl >= 0:
            expect[sl] = ref["conv_state"][0]
            used.append(sl)
    got_pool = np64(pool)
    assert np.array_equal(got_pool[used], expect[used]), "new convolution states"
    untouched = [i for i in range(pool_size) if i not in used]
    assert np.array_equal(got_pool[untouched], p0[untouched]), "slots no sequence uses must not change"


def test_prepare_varlen_mixed_lengths_slots_and_starts():
    lens = [5, 0, 70, 1, 2, 33, 40, 3]
    slots = [4, 0, 7, -1, 2, 9, 1, 5]
    init = [1, 1, 0, 1, 1, 1, 0, 1]
    varlen_case(lens, 3, 64, 64, 10, slots, init)


def test_prepare_varlen_fp32_default_slots():
    varlen_case([31, 1, 64, 2, 0, 7], 2, 16, 64, 6, None, None, dtype=torch.float32, wid=301)


def test_prepare_varlen_decode_batch():
    # a serving decode step: 64 sequences of one token, states in a 100-slot pool
    rng = np.random.default_rng(9)
    slots = rng.permutation(100)[:64].astype(np.int32).tolist()
    varlen_case([1] * 64, 4, 64, 64, 100, slots, None, wid=302)


@pytest.mark.parametrize("hi", [3, 9], ids=["tile2or4", "tile8"])
def test_prepare_varlen_short_sequences(hi):
    # short prompts: tiles shrink to the mean length (a power of two below 32), so sequence starts
    # fall inside tiles and sequences run across tile edges
    rng = np.random.default_rng(hi)
    lens = rng.integers(0, hi + 1, size=40).tolist()
    slots = rng.permutation(48)[:40].astype(np.int32).tolist()
    init = rng.integers(0, 2, size=40).tolist()
    varlen_case(lens, 2, 64, 64, 48, slots, init, wid=306 + hi)


def test_prepare_varlen_empty_sequences_and_one_token_tiles():
    # mostly empty sequences pull the mean length below 1: one-token tiles, so the 3- and 5-token
    # sequences run across tiles (their windows and new states come from the tokens before each tile)
    lens = [0, 0, 3, 0, 0, 0, 1, 0, 0, 5, 0, 0]
    slots = [0, 1, 2, 3, 4, -1, 6, 7, 8, 9, 10, 11]
    init = [1, 0, 1, 1, 0, 1, 1, 1, 1, 0, 1, 1]
    varlen_case(lens, 2, 64, 64, 12, slots, init, wid=320)


def test_prepare_varlen_single_sequence_equals_dense():
    d = gi.prep_inputs(1, 150, 2, 64, 64, wid=303, device=DEV)
    dense_state = torch.empty_like(d["conv_state"])
    dense = run(d, state_out=dense_state)
    pool = d["conv_state"].clone()
    x = {kk: (t[0] if kk in ("xq", "xk", "xv", "a_raw", "b_raw") else t) for kk, t in d.items()}
    packed = gdn.prepare_varlen(x["xq"], x["xk"], x["xv"], x["conv_weight"], x["a_raw"], x["b_raw"], [0, 150], pool,
                                decay_rate=x["decay_rate"], gate_bias=x["gate_bias"])
    torch.cuda.synchronize()
    for i, name in enumerate(("q", "k", "v", "g", "beta")):
        assert torch.equal(packed[i], dense[i][0]), name
    assert torch.equal(pool, dense_state)


def test_wrong_sized_buffers_are_refused_before_any_launch():
    # the C ABI takes bare pointers; the binding checks every shape so that a buffer of another call's
    # size is never read or written past its end
    print("[case] wrong-sized buffers", flush=True)
    d = gi.prep_inputs(1, 40, 2, 64, 64, wid=304, device=DEV)
    small = gi.prep_inputs(1, 8, 2, 64, 64, wid=305, device=DEV)
    outs = tuple(torch.empty_like(small[kk]) for kk in ("xq", "xk", "xv", "a_raw", "b_raw"))
    with pytest.raises(ValueError, match="shape"):
        gdn.prepare(d["xq"], d["xk"], d["xv"], d["conv_weight"], d["a_raw"], d["b_raw"], outs=outs)
    with pytest.raises(ValueError, match="shape"):
        gdn.prepare(d["xq"], d["xk"], small["xv"], d["conv_weight"], d["a_raw"], d["b_raw"])
    q, k, v = (d["xq"], d["xk"], d["xv"])
    g = torch.zeros(d["a_raw"].shape, device=DEV)
    with pytest.raises(ValueError, match="shape"):
        gdn.chunk_prefill(q, k, v, g, g, out=torch.empty((1, 8, 2, 64), device=DEV))
    with pytest.raises(ValueError, match="shape"):
        gdn.chunk_backward(q, k, v, g, g, torch.zeros((1, 40, 2, 64), device=DEV),
                           outs=tuple(torch.empty((1, 8, 2, 64), device=DEV) for _ in range(6)))
