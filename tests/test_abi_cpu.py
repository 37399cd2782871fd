"""The C-ABI library loads, exports what include/gdn.h declares, and rejects bad
arguments on the host before touching the GPU (CPU only: no kernel runs)."""
import os
import re

import pytest

import hybrid_linear_attention_gated_amd as gdn

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "gdn.h")
OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WS = 0, 1, 2, 3, 4, 5, 6
BF16, F32 = gdn.GDN_BF16, gdn.GDN_F32


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"GDN_API\s+[\w\s\*]+?\b(gdn_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(gdn.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = gdn.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert gdn.gdn_version() == 7


def test_status_strings():
    for code in range(9):
        assert gdn.gdn_status_string(code).startswith(gdn.STATUS[code])
    assert "rule" in gdn.gdn_status_string(3)
    assert gdn.gdn_status_string(99) == "unknown gdn_status"


# fake, never dereferenced device addresses (validation is host-only)
A = 1 << 32


def addr(i, size=1 << 30):
    return A + i * size


def prefill(**kw):
    args = dict(q=addr(0), k=addr(1), v=addr(2), g=addr(3), beta=addr(4), s0=None, o=addr(5),
                sf=addr(6), B=1, T=65536, H=2, dk=64, dv=64, chunk=64, dt=BF16, ws=addr(7),
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return gdn.gdn_chunk_prefill(args["q"], args["k"], args["v"], args["g"], args["beta"], args["s0"],
                                 args["o"], args["sf"], args["B"], args["T"], args["H"], args["dk"],
                                 args["dv"], args["chunk"], args["dt"], args["ws"], args["ws_bytes"],
                                 args["stream"])


def decode(**kw):
    args = dict(q=addr(0), k=addr(1), v=addr(2), g=addr(3), beta=addr(4), st=addr(5), o=addr(6),
                N=4, H=2, dk=64, dv=64, dt=BF16, stream=None)
    args.update(kw)
    return gdn.gdn_decode_step(args["q"], args["k"], args["v"], args["g"], args["beta"], args["st"],
                               args["o"], args["N"], args["H"], args["dk"], args["dv"], args["dt"],
                               args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(o=None), NULL), (dict(sf=None), NULL), (dict(beta=None), NULL),
    (dict(B=0), SHAPE), (dict(H=-1), SHAPE), (dict(T=-5), SHAPE), (dict(chunk=0), SHAPE),
    (dict(dk=32), UNSUP), (dict(dv=96), UNSUP), (dict(chunk=128), UNSUP), (dict(dt=7), UNSUP),
    (dict(q=addr(0) + 8), ALIGN), (dict(sf=addr(6) + 4), ALIGN), (dict(ws=addr(7) + 2), ALIGN),
    (dict(o=addr(0)), ALIAS), (dict(o=addr(2) + 64), ALIAS), (dict(sf=addr(1)), ALIAS),
    (dict(sf=addr(5)), ALIAS), (dict(s0=addr(8), sf=addr(8) + 256), ALIAS),
    (dict(s0=addr(5)), ALIAS),
    (dict(ws=None), WS), (dict(ws_bytes=1024), WS), (dict(ws=addr(4)), ALIAS),
])
def test_prefill_rejects(kw, code):
    assert prefill(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(st=None), NULL), (dict(o=None), NULL),
    (dict(N=-1), SHAPE), (dict(H=0), SHAPE), (dict(dk=8), UNSUP), (dict(dt=3), UNSUP),
    (dict(st=addr(5) + 4), ALIGN), (dict(o=addr(1)), ALIAS), (dict(st=addr(2)), ALIAS),
    (dict(o=addr(5) + 1024), ALIAS),
])
def test_decode_rejects(kw, code):
    assert decode(**kw) == code


def test_decode_rejects_a_grid_past_the_launch_limit():
    """128-wide states take eight wavefronts per (sequence, head): N H 8 must stay below 2^31."""
    assert decode(N=1 << 26, H=5, dk=128, dv=128) == SHAPE


def test_decode_zero_sequences_is_a_no_op():
    assert decode(N=0, q=None, k=None) == OK


def test_workspace_size():
    # one sequence piece: everything stays on chip
    assert gdn.gdn_chunk_prefill_workspace_size(1, 128, 32, 64, 64, 64, BF16) == 0
    # long sequences with few heads are split into pieces; scratch holds the piece maps
    # [DK][DV+DK] and start states [DK][DV], fp32, a few tens of MB at most
    w = gdn.gdn_chunk_prefill_workspace_size(1, 65536, 32, 64, 64, 64, BF16)
    assert 0 < w < 64 << 20
    # 128-wide heads also keep every chunk's T diag(b) fragments: 4 KiB per 32-token chunk and head
    # (10 pieces of 205 chunks for 24 heads)
    maps, starts = 24 * 9 * 128 * 256 * 4, 24 * 10 * 128 * 128 * 4
    assert gdn.gdn_chunk_prefill_workspace_size(1, 65536, 24, 128, 128, 64, BF16) == maps + starts + 24 * 2048 * 4096
    # fp32 inputs and the VALU shapes need none
    assert gdn.gdn_chunk_prefill_workspace_size(1, 64, 2, 16, 16, 16, F32) == 0
    assert gdn.gdn_chunk_prefill_workspace_size(1, 65536, 2, 64, 64, 16, BF16) == 0
    # rejected arguments and T = 0 need nothing
    assert gdn.gdn_chunk_prefill_workspace_size(1, 64, 2, 48, 64, 64, BF16) == 0
    assert gdn.gdn_chunk_prefill_workspace_size(1, 0, 2, 64, 64, 64, BF16) == 0


def test_rule_entry_points_validate_the_rule():
    args = dict(q=addr(0), k=addr(1), v=addr(2), g=addr(3), beta=addr(4), s0=None, o=addr(5),
                sf=addr(6), B=1, T=65536, H=2, dk=64, dv=64, chunk=64, dt=BF16, ws=addr(7),
                ws_bytes=1 << 30, stream=None)
    pre = lambda rule, **kw: gdn.gdn_chunk_prefill_rule(
        rule, *[dict(args, **kw)[n] for n in ("q", "k", "v", "g", "beta", "s0", "o", "sf", "B", "T", "H",
                                              "dk", "dv", "chunk", "dt", "ws", "ws_bytes", "stream")])
    assert pre(2) == UNSUP and pre(-1) == UNSUP
    # the rule is checked first, then the same argument checks as gdn_chunk_prefill
    for rule in (gdn.GDN_RULE_GATED_DELTA, gdn.GDN_RULE_GATED_DECAY):
        assert pre(rule, q=None) == NULL and pre(rule, dk=32) == UNSUP and pre(rule, o=addr(0)) == ALIAS
    dec = lambda rule, **kw: gdn.gdn_decode_step_rule(
        rule, *[dict(dict(q=addr(0), k=addr(1), v=addr(2), g=addr(3), beta=addr(4), st=addr(5), o=addr(6),
                          N=4, H=2, dk=64, dv=64, dt=BF16, stream=None), **kw)[n]
                for n in ("q", "k", "v", "g", "beta", "st", "o", "N", "H", "dk", "dv", "dt", "stream")])
    assert dec(5) == UNSUP
    assert dec(gdn.GDN_RULE_GATED_DECAY, st=addr(2)) == ALIAS
    assert dec(gdn.GDN_RULE_GATED_DECAY, N=0, q=None) == OK


def test_decode_slots_validation():
    base = dict(q=addr(0), k=addr(1), v=addr(2), g=addr(3), beta=addr(4), pool=addr(5), slots=addr(6),
                P=10, o=addr(7), N=4, H=2, dk=64, dv=64, dt=BF16, stream=None)

    def call(rule=gdn.GDN_RULE_GATED_DELTA, **kw):
        a = dict(base, **kw)
        return gdn.gdn_decode_step_slots(rule, a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"],
                                         a["slots"], a["P"], a["o"], a["N"], a["H"], a["dk"], a["dv"],
                                         a["dt"], a["stream"])
    assert call(slots=None) == NULL
    assert call(pool=None) == NULL
    assert call(P=-1) == SHAPE
    assert call(rule=3) == UNSUP
    assert call(slots=addr(6) + 4) == ALIGN
    assert call(o=addr(6)) == ALIAS            # output over the slot table
    assert call(pool=addr(6) - 1024) == ALIAS  # pool running into the slot table
    assert call(N=0, slots=None, q=None) == OK


def test_varlen_validation():
    import numpy as np
    cu = np.array([0, 100, 100, 350], dtype=np.int32)

    def call(cu=cu, slots=None, init=None, P=8, dt=BF16, dk=64, dv=64, chunk=64, T=350, ws_bytes=1 << 30,
             rule=gdn.GDN_RULE_GATED_DELTA, o=addr(5), pool=addr(6), ws=addr(7)):
        S = len(cu) - 1
        return gdn.gdn_chunk_prefill_varlen(rule, addr(0), addr(1), addr(2), addr(3), addr(4),
                                            None if cu is None else cu.ctypes.data, S, T, pool, P,
                                            None if slots is None else slots.ctypes.data,
                                            None if init is None else init.ctypes.data, o, 2, dk, dv, chunk, dt,
                                            ws, ws_bytes, None)
    assert call(rule=4) == UNSUP
    assert call(dt=7) == UNSUP and call(dk=32) == UNSUP and call(chunk=8) == UNSUP
    # fp32 q/k/v and the 16-wide shapes go to the VALU kernel, whose workspace is a 4 x S int table
    assert call(dt=F32, ws_bytes=255) == WS and call(dk=16, chunk=16, ws=None) == WS
    assert call(T=351) == SHAPE                                   # offsets must end at T_total
    assert call(cu=np.array([0, 100, 90, 350], dtype=np.int32)) == SHAPE  # decreasing offsets
    assert call(cu=np.array([5, 100, 350], dtype=np.int32)) == SHAPE      # must start at 0
    assert call(P=2) == SHAPE                                     # slot s = s needs pool_size >= S
    assert call(slots=np.array([1, 8, 0], dtype=np.int32)) == SHAPE       # slot out of range
    assert call(slots=np.array([1, -2, 0], dtype=np.int32)) == SHAPE
    assert call(slots=np.array([3, 5, 3], dtype=np.int32)) == ALIAS       # one state, two sequences
    assert call(pool=None) == NULL
    assert call(ws_bytes=16) == WS and call(ws=None) == WS
    assert call(o=addr(0)) == ALIAS and call(pool=addr(4)) == ALIAS
    need = gdn.gdn_chunk_prefill_varlen_workspace_size(cu.ctypes.data, 3, 2, 64, 64, 64, BF16)
    assert 0 < need < 1 << 20
    assert gdn.gdn_chunk_prefill_varlen_workspace_size(cu.ctypes.data, 3, 2, 16, 64, 64, BF16) == 256
    assert gdn.gdn_chunk_prefill_varlen_workspace_size(cu.ctypes.data, 3, 2, 64, 64, 64, F32) == 256
    assert gdn.gdn_chunk_prefill_varlen_workspace_size(cu.ctypes.data, 3, 2, 32, 64, 64, F32) == 0
    assert call(cu=np.array([0], dtype=np.int32), T=0) == OK      # no sequences: nothing to do


def prepare_call(**kw):
    args = dict(xq=addr(0), xk=addr(1), xv=addr(2), w=addr(3), a=addr(4), b=addr(5), rate=None, bias=None,
                s_in=None, s_out=None, q=addr(6), k=addr(7), v=addr(8), g=addr(9), beta=addr(10),
                B=1, T=65536, H=32, dk=64, dv=64, dt=BF16, stream=None)
    args.update(kw)
    return gdn.gdn_prepare(*[args[n] for n in ("xq", "xk", "xv", "w", "a", "b", "rate", "bias", "s_in", "s_out",
                                                "q", "k", "v", "g", "beta", "B", "T", "H", "dk", "dv", "dt",
                                                "stream")])


@pytest.mark.parametrize("kw,code", [
    (dict(w=None), NULL), (dict(xq=None), NULL), (dict(beta=None), NULL), (dict(v=None), NULL),
    (dict(B=0), SHAPE), (dict(T=-1), SHAPE), (dict(H=0), SHAPE), (dict(T=1 << 30, H=1 << 12), SHAPE),
    (dict(dk=32), UNSUP), (dict(dv=96), UNSUP), (dict(dt=5), UNSUP),
    (dict(xk=addr(1) + 8), ALIGN), (dict(s_out=addr(11) + 4), ALIGN), (dict(rate=addr(12) + 2), ALIGN),
    (dict(q=addr(0)), ALIAS), (dict(v=addr(6) + 1024), ALIAS), (dict(g=addr(4)), ALIAS),
    (dict(beta=addr(9)), ALIAS), (dict(s_out=addr(3)), ALIAS), (dict(s_in=addr(11), s_out=addr(11) + 16), ALIAS),
    (dict(k=addr(12), rate=addr(12)), ALIAS), (dict(s_in=addr(11), q=addr(11)), ALIAS),
])
def test_prepare_rejects(kw, code):
    assert prepare_call(**kw) == code


def test_prepare_nothing_to_do_is_a_no_op():
    # T = 0 with no state to carry: validated, nothing queued (no GPU needed)
    assert prepare_call(T=0, xq=None, xk=None, xv=None, a=None, b=None, q=None, k=None, v=None, g=None,
                        beta=None) == OK


def backward_call(**kw):
    args = dict(rule=0, q=addr(0), k=addr(1), v=addr(2), g=addr(3), beta=addr(4), s0=None, do=addr(5), dsf=None,
                dq=addr(6), dk=addr(7), dv=addr(8), dg=addr(9), db=addr(10), ds0=None, B=1, T=8192, H=4, dk_=64,
                dv_=64, dt=BF16, ws=addr(11, 1 << 34), ws_bytes=1 << 33, stream=None)
    args.update(kw)
    return gdn.gdn_chunk_backward(*[args[n] for n in ("rule", "q", "k", "v", "g", "beta", "s0", "do", "dsf", "dq",
                                                      "dk", "dv", "dg", "db", "ds0", "B", "T", "H", "dk_", "dv_",
                                                      "dt", "ws", "ws_bytes", "stream")])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(do=None), NULL), (dict(dbeta=None) if False else dict(db=None), NULL),
    (dict(B=0), SHAPE), (dict(T=-1), SHAPE), (dict(rule=3), UNSUP), (dict(dk_=128), UNSUP), (dict(dt=5), UNSUP),
    (dict(dq=addr(6) + 4), ALIGN), (dict(ws=addr(11, 1 << 34) + 8), ALIGN),
    (dict(dq=addr(0)), ALIAS), (dict(dk=addr(6) + 256), ALIAS), (dict(ds0=addr(3)), ALIAS),
    (dict(dv=addr(11, 1 << 34)), ALIAS), (dict(ws=None), WS), (dict(ws_bytes=1024), WS),
])
def test_backward_rejects(kw, code):
    assert backward_call(**kw) == code


def test_backward_workspace_size():
    assert gdn.gdn_chunk_backward_workspace_size(1, 8192, 4, 64, 64, BF16) > 4 * 256 * 64 * 64 * 4 * 4
    assert gdn.gdn_chunk_backward_workspace_size(1, 8192, 4, 128, 128, BF16) > 4 * 256 * 128 * 128 * 4 * 4
    assert gdn.gdn_chunk_backward_workspace_size(1, 8192, 4, 16, 16, BF16) == 0
    assert gdn.gdn_chunk_backward_workspace_size(1, 8192, 4, 64, 128, BF16) == 0
    assert gdn.gdn_chunk_backward_workspace_size(0, 8192, 4, 64, 64, BF16) == 0
    # nothing to compute: T = 0 without an initial-state gradient is accepted without a GPU
    assert backward_call(T=0, q=None, k=None, v=None, g=None, beta=None, do=None, dq=None, dk=None, dv=None,
                         dg=None, db=None) == OK


def prepare_varlen_call(**kw):
    import numpy as np
    cu = kw.pop("cu", np.array([0, 5, 5, 12], dtype=np.int32))
    slots = kw.pop("slots", None)
    S = kw.pop("S", len(cu) - 1)
    args = dict(xq=addr(0), xk=addr(1), xv=addr(2), w=addr(3), a=addr(4), b=addr(5), rate=None, bias=None,
                T=int(cu[-1]) if len(cu) else 0, pool=addr(6), pool_size=4, init=None, q=addr(7), k=addr(8),
                v=addr(9), g=addr(10), beta=addr(11), H=2, dk=64, dv=64, dt=BF16, ws=addr(12), ws_bytes=4096,
                stream=None)
    args.update(kw)
    cup = cu.ctypes.data if len(cu) else None
    slp = None if slots is None else slots.ctypes.data
    return gdn.gdn_prepare_varlen(args["xq"], args["xk"], args["xv"], args["w"], args["a"], args["b"], args["rate"],
                                  args["bias"], cup, S, args["T"], args["pool"], args["pool_size"], slp, args["init"],
                                  args["q"], args["k"], args["v"], args["g"], args["beta"], args["H"], args["dk"],
                                  args["dv"], args["dt"], args["ws"], args["ws_bytes"], args["stream"])


def test_prepare_varlen_validation():
    import numpy as np
    assert prepare_varlen_call(ws=None) == WS
    assert prepare_varlen_call(ws_bytes=8) == WS
    assert prepare_varlen_call(cu=np.array([0, 5, 4, 12], dtype=np.int32)) == SHAPE      # decreasing offsets
    assert prepare_varlen_call(cu=np.array([1, 5, 5, 12], dtype=np.int32)) == SHAPE      # not from 0
    assert prepare_varlen_call(T=13) == SHAPE                                             # cu[S] != T_total
    assert prepare_varlen_call(pool_size=2) == SHAPE                                      # default slots need S slots
    assert prepare_varlen_call(slots=np.array([0, 4, 1], dtype=np.int32)) == SHAPE        # slot out of range
    assert prepare_varlen_call(slots=np.array([1, 1, -1], dtype=np.int32)) == ALIAS       # repeated slot
    assert prepare_varlen_call(pool=None) == NULL
    # no slot in use: the pool may be NULL (validation then stops at the missing workspace, no launch)
    assert prepare_varlen_call(pool=None, slots=np.array([-1, -1, -1], dtype=np.int32), ws=None) == WS
    assert prepare_varlen_call(w=None) == NULL
    assert prepare_varlen_call(dk=32) == UNSUP
    assert prepare_varlen_call(q=addr(0)) == ALIAS
    assert prepare_varlen_call(pool=addr(3)) == ALIAS
    assert prepare_varlen_call(ws=addr(6)) == ALIAS
    assert prepare_varlen_call(xk=addr(1) + 4) == ALIGN
    assert gdn.gdn_prepare_varlen_workspace_size(0) == 0
    assert gdn.gdn_prepare_varlen_workspace_size(3) >= 40
    # no sequences: nothing to do
    assert prepare_varlen_call(cu=np.array([0], dtype=np.int32), S=0, T=0) == OK


def prepare_decode_call(**kw):
    args = dict(rule=0, xq=addr(0), xk=addr(1), xv=addr(2), w=addr(3), a=addr(4), b=addr(5), rate=None, bias=None,
                conv=addr(6), state=addr(7), o=addr(8), N=256, H=32, dk=64, dv=64, dt=BF16, stream=None)
    args.update(kw)
    return gdn.gdn_prepare_decode_step(*[args[n] for n in ("rule", "xq", "xk", "xv", "w", "a", "b", "rate", "bias",
                                                           "conv", "state", "o", "N", "H", "dk", "dv", "dt",
                                                           "stream")])


@pytest.mark.parametrize("kw,code", [
    (dict(rule=2), UNSUP), (dict(H=0), SHAPE), (dict(N=-1), SHAPE), (dict(dk=16, dv=16), UNSUP),
    (dict(dk=64, dv=128), UNSUP), (dict(dt=5), UNSUP), (dict(N=1 << 30, H=4), SHAPE),
    (dict(xq=None), NULL), (dict(conv=None), NULL), (dict(state=None), NULL), (dict(o=None), NULL),
    (dict(w=None), NULL), (dict(b=None), NULL),
    (dict(xk=addr(1) + 8), ALIGN), (dict(state=addr(7) + 4), ALIGN), (dict(bias=addr(9) + 2), ALIGN),
    (dict(o=addr(7) + 256), ALIAS), (dict(conv=addr(0)), ALIAS), (dict(state=addr(6) + 64), ALIAS),
    (dict(o=addr(4)), ALIAS), (dict(rate=addr(8)), ALIAS),
])
def test_prepare_decode_rejects(kw, code):
    assert prepare_decode_call(**kw) == code


def test_prepare_decode_no_sequences_is_a_no_op():
    assert prepare_decode_call(N=0, xq=None, xk=None, xv=None, conv=None, state=None, o=None) == OK


def test_noalloc_validates_like_the_workspace_call():
    """gdn_chunk_prefill_noalloc rejects what gdn_chunk_prefill_rule rejects, before it looks up its
    scratch on the device (so these run without a GPU)."""
    def call(rule=0, dk=64, B=1, T=1000, q=addr(0), o=addr(5), dt=BF16):
        return gdn.gdn_chunk_prefill_noalloc(rule, q, addr(1), addr(2), addr(3), addr(4), None, o, addr(6), B, T, 2,
                                             dk, 64, 64, dt, None)
    assert call(rule=9) == UNSUP
    assert call(dk=32) == UNSUP
    assert call(dt=5) == UNSUP
    assert call(B=0) == SHAPE
    assert call(T=-1) == SHAPE


def prepare_prefill_call(**kw):
    args = dict(rule=0, xq=addr(0), xk=addr(1), xv=addr(2), w=addr(3), a=addr(4), b=addr(5), rate=None, bias=None,
                cin=None, cout=None, s0=None, o=addr(6), sf=addr(7), B=1, T=4096, H=4, dk=64, dv=64, chunk=64,
                dt=BF16, ws=addr(8), ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return gdn.gdn_prepare_chunk_prefill(*[args[n] for n in ("rule", "xq", "xk", "xv", "w", "a", "b", "rate", "bias",
                                                             "cin", "cout", "s0", "o", "sf", "B", "T", "H", "dk", "dv",
                                                             "chunk", "dt", "ws", "ws_bytes", "stream")])


@pytest.mark.parametrize("kw,code", [
    (dict(rule=2), UNSUP), (dict(dt=F32), UNSUP), (dict(dk=64, dv=128), UNSUP), (dict(dk=16, dv=16), UNSUP),
    (dict(chunk=16), UNSUP), (dict(B=0), SHAPE), (dict(T=-1), SHAPE), (dict(H=0), SHAPE),
    (dict(xq=None), NULL), (dict(w=None), NULL), (dict(sf=None), NULL), (dict(o=None), NULL), (dict(b=None), NULL),
    (dict(xk=addr(1) + 8), ALIGN), (dict(cin=addr(9) + 4), ALIGN), (dict(sf=addr(7) + 4), ALIGN),
    (dict(o=addr(0)), ALIAS), (dict(sf=addr(3)), ALIAS), (dict(cout=addr(2) + 64), ALIAS),
    (dict(cin=addr(9), cout=addr(9) + 16), ALIAS), (dict(s0=addr(10), sf=addr(10) + 256), ALIAS),
    (dict(ws=addr(0)), ALIAS), (dict(ws=None), WS), (dict(ws_bytes=64), WS),
])
def test_prepare_prefill_rejects(kw, code):
    assert prepare_prefill_call(**kw) == code


def test_prepare_prefill_workspace_size():
    n = gdn.gdn_prepare_chunk_prefill_workspace_size(1, 65536, 32, 64, 64, 64, BF16)
    assert n == gdn.gdn_chunk_prefill_workspace_size(1, 65536, 32, 64, 64, 32, BF16) > 0
    assert gdn.gdn_prepare_chunk_prefill_workspace_size(1, 65536, 32, 64, 64, 64, F32) == 0
    assert gdn.gdn_prepare_chunk_prefill_workspace_size(1, 100, 2, 64, 64, 64, BF16) == 0
