#!/usr/bin/env python3
"""Benchmark of the GDN token mixer on one MI355X.

One step = one pass of the whole hot path on synthetic inputs already resident
in HBM:
  * prefill: one gdn_chunk_prefill call on the 1B-shaped 64K workload
    (B=1, H=32, T=65536, d_k=d_v=64, chunk 64, bf16 q/k/v, fp32 gates and
    state, start state carried in, final state returned);
  * decode: 16 consecutive gdn_decode_step calls on 256 sequences
    (H=32, d=64, fp32 per-sequence state).
`value` is the prefill throughput in tokens/s (65536 tokens per call);
decode is reported beside it in GB/s of state traffic.

Each component is timed with HIP events recorded on the stream its kernels
are launched on (the current torch stream).  `roofline` describes the
prefill call (HBM-bound: algorithmic bytes / call time vs 8 TB/s), with the
useful MFMA work (chunk-form FLOPs, no precision splits) as a fraction of the
2.5 PFLOP/s bf16 dense peak next to it.  `roofline.traffic` is the HBM byte count of one
call from the committed FETCH_SIZE/WRITE_SIZE counter summary, reported only
while the kernel sources still hash to the digest recorded with it (else
null).  Decode is also timed cold: a 1 GiB buffer is read before every step
(outside the timed events) so the state cannot come from the 256 MB
last-level cache.  `cpu_baseline` is the fp64 oracle (tests only, never the
product path) timed on the host cores on the same 64K prefill workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

# Per token-head figures for d_k = d_v = 64, chunk 64.
#   bytes: q, k, v bf16 (3 * 64 * 2) + g, beta fp32 (8) + o fp32 (64 * 4) = 648
#   useful FLOPs: C (6 d_k + 4 d_v) + 6 d_k d_v + C^2 / 3 = 66,901 (chunk-form
#   contractions K K^T, Q K^T, U, W, P Delta, W St, Q St, K^T Delta and the
#   forward substitution)
BYTES_PER_TOKEN_HEAD = 648
FLOPS_PER_TOKEN_HEAD = 64 * (6 * 64 + 4 * 64) + 6 * 64 * 64 + 64 * 64 // 3
# the most useful MFMA work per second the HBM floor allows, as a fraction of the bf16 peak:
# (FLOPs / bytes) x 8 TB/s / 2.5 PFLOP/s = 103.2 x 8e12 / 2.5e15 = 0.330
CEILING_MFMA_FRAC = FLOPS_PER_TOKEN_HEAD / BYTES_PER_TOKEN_HEAD * HBM_PEAK_GBPS * 1e9 / (BF16_PEAK_TFLOPS * 1e12)
# the same at d_k = d_v = 128 (one 64K call of the 3B-shaped chain): 3 * 128 * 2 + 8 + 128 * 4 bytes,
# C (6 d_k + 4 d_v) + 6 d_k d_v + C^2 / 3 FLOPs
BYTES_PER_TOKEN_HEAD_128 = 3 * 128 * 2 + 8 + 128 * 4
FLOPS_PER_TOKEN_HEAD_128 = 64 * (6 * 128 + 4 * 128) + 6 * 128 * 128 + 64 * 64 // 3
# decode, per (sequence, head) per step: state read + write (2 * 4 * 64 * 64),
# q, k, v bf16 (3 * 64 * 2), g, beta (8), o fp32 (64 * 4)
DECODE_BYTES_PER_SEQ_HEAD = 2 * 4 * 64 * 64 + 3 * 64 * 2 + 8 + 64 * 4
# preparation ahead of the mixer, per token-head: raw q/k/v projections read and q/k/v written, bf16
# (2 * 3 * 64 * 2), gate and write-strength logits read and g, beta written, fp32 (4 * 4) = 784; per
# channel once per call: convolution weights (4 * 4) and, per sequence, the carried state read and
# written (2 * 3 * 4)
PREP_BYTES_PER_TOKEN_HEAD = 2 * 3 * 64 * 2 + 4 * 4
# gradients (d_k = d_v = 64, chunks of 32 tokens), multiply-adds per chunk and head of the kernels'
# products: keyside once, in the map pass, which stores it for the gradient pass (P, K K^T, W:
# 3 C^2 d + C^3/6 = 202,411), map (X, R, F: C^2 d + 2 C d^2 = 327,680), scan (d^3 = 262,144), gradients
# (Delta, K Y, dDelta, dP, dQ, dq, dW, T^T dW, T^T dDelta, dT, dA, dK: 10 C^2 d + 5 C d^2 + 2 C^3 =
# 1,441,792); 2 FLOPs each, per token-head = / 32
BWD_FLOPS_PER_TOKEN_HEAD = 2 * (202411 + 327680 + 262144 + 1441792) // 32
FP32_VALU_PEAK_TFLOPS = 157.3
COPY_BYTES = 4 << 30  # far larger than the 256 MB last-level cache
FLUSH_BYTES = 1 << 30
CSRC = os.path.join(ROOT, "hybrid_linear_attention_gated_amd", "csrc")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_1b_64k_decode_n256_h32.md")


def recorded_traffic(kind):
    """Counter-measured HBM bytes for `kind` ('prefill', 'prepare' and 'prepared' -- the prefill
    from the raw projections in one pass -- per 64K call, 'decode' per step, 'fused' per one-launch
    decode step of the 256-sequence batch) from the committed summary, or None when the kernel
    sources no longer match the recorded digest."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            fields = dict(line.strip().split(": ", 1) for line in f if line.strip().startswith(kind + "-"))
        d = hashlib.sha256()
        for name in fields[kind + "-sources"].split():
            with open(os.path.join(CSRC, name), "rb") as src:
                d.update(src.read())
        if d.hexdigest() != fields[kind + "-source-sha256"]:
            return None
        unit = "step" if kind == "decode" else "call"
        return int(fields[f"{kind}-traffic-bytes-per-{unit}"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=65536,
                    help="tokens of the 64K workload the oracle is timed on")
    ap.add_argument("--backward-workload", choices=["1b_8k", "1b_64k"], default="1b_8k",
                    help="workload of the backward leg (the JSON line reports 1b_8k)")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "copy", "prepare", "backward"], default="all",
                    help="run one component (for profiling); 'copy' runs a plain 4 GiB device copy "
                         "used to calibrate the HBM byte counters; the JSON line needs 'all'")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (--gpus 1): heads and the sequences of a batch shard "
              "over GPUs with no exchange inside the mixer, so a multi-GPU run would repeat the "
              "one-GPU kernels on smaller shares.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gdn_inputs as gi
    import hybrid_linear_attention_gated_amd as gdn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.only == "copy":
        # counter calibration (each copy reads and writes exactly COPY_BYTES) and the device's
        # achievable read + write bandwidth on a buffer far larger than the last-level cache
        src = torch.ones(COPY_BYTES // 4, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.warmup + args.steps)]
        for a, b in ev:
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev[args.warmup:]]
        gbps = 2 * COPY_BYTES / (sum(ms) / len(ms) * 1e-3) / 1e9
        print(json.dumps({"only": "copy", "bytes_per_copy": COPY_BYTES, "copies": len(ev),
                          "read_plus_write_GBps": round(gbps, 1)}))
        return

    # ---- inputs (resident before timing) ----
    w = gi.WORKLOADS["1b_64k"]
    pre = gi.workload_inputs("1b_64k", device=dev)
    out = torch.empty((w.B, w.T, w.H, w.dv), device=dev, dtype=torch.float32)
    fin = torch.empty((w.B, w.H, w.dk, w.dv), device=dev, dtype=torch.float32)
    wsz = gdn.workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.chunk, gdn.GDN_BF16)
    ws = torch.empty(max(wsz, 1), device=dev, dtype=torch.uint8)

    dw = gi.WORKLOADS["decode"]
    steps_in = [gi.decode_inputs(dw.B, dw.H, dw.dk, dw.dv, s, device=dev) for s in range(dw.calls)]
    state0 = gi.decode_state(dw.B, dw.H, dw.dk, dw.dv, device=dev)
    state = state0.clone()
    dout = torch.empty((dw.B, dw.H, dw.dv), device=dev, dtype=torch.float32)

    # input preparation ahead of the mixer (short convolution, SiLU, q/k norm, gates) on the same
    # 64K shape and on the decode batch (one token per sequence, convolution state carried in place)
    pin = gi.prep_inputs(w.B, w.T, w.H, w.dk, w.dv, wid=200, device=dev)
    pouts = (torch.empty_like(pin["xq"]), torch.empty_like(pin["xk"]), torch.empty_like(pin["xv"]),
             torch.empty((w.B, w.T, w.H), device=dev, dtype=torch.float32),
             torch.empty((w.B, w.T, w.H), device=dev, dtype=torch.float32))
    pstate = torch.empty_like(pin["conv_state"])
    din = gi.prep_inputs(dw.B, 1, dw.H, dw.dk, dw.dv, wid=201, device=dev)
    dstate0 = din["conv_state"].clone()
    # the same decode step through the serving pool: 256 one-token sequences, states in a 512-slot pool
    import numpy as np
    pcu = np.arange(dw.B + 1, dtype=np.int32)
    pslots = np.random.default_rng(12).permutation(2 * dw.B)[:dw.B].astype(np.int32)
    ppool = torch.zeros((2 * dw.B, din["conv_state"].shape[1], 3), device=dev, dtype=torch.float32)
    pflat = {kk: din[kk][:, 0].contiguous() for kk in ("xq", "xk", "xv", "a_raw", "b_raw")}
    pool_outs = tuple(torch.empty_like(pflat[kk]) for kk in ("xq", "xk", "xv", "a_raw", "b_raw"))
    pws = torch.empty(max(gdn.gdn_prepare_varlen_workspace_size(dw.B), 1), device=dev, dtype=torch.uint8)

    def prepare_decode_pool():
        gdn.prepare_varlen(pflat["xq"], pflat["xk"], pflat["xv"], din["conv_weight"], pflat["a_raw"], pflat["b_raw"],
                           pcu, ppool, slots=pslots, decay_rate=din["decay_rate"], gate_bias=din["gate_bias"],
                           outs=pool_outs, workspace=pws)

    # the same decode step (preparation + state update) fused into one launch, and as two launches
    fstate = gi.decode_state(dw.B, dw.H, dw.dk, dw.dv, wid=202, device=dev)
    fconv = din["conv_state"].clone()
    fout = torch.empty((dw.B, dw.H, dw.dv), device=dev, dtype=torch.float32)
    souts = tuple(torch.empty((dw.B, 1) + tuple(t.shape[1:]), device=dev, dtype=t.dtype) for t in pool_outs)

    def decode_fused():
        gdn.prepare_decode_step(pflat["xq"], pflat["xk"], pflat["xv"], din["conv_weight"], pflat["a_raw"],
                                pflat["b_raw"], fconv, fstate, decay_rate=din["decay_rate"],
                                gate_bias=din["gate_bias"], out=fout)

    def decode_separate():
        q, k, v, g, b = gdn.prepare(din["xq"], din["xk"], din["xv"], din["conv_weight"], din["a_raw"], din["b_raw"],
                                    decay_rate=din["decay_rate"], gate_bias=din["gate_bias"], conv_state=fconv,
                                    conv_state_out=fconv, outs=souts)
        gdn.decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], b[:, 0], fstate, out=fout)

    def prepare():
        gdn.prepare(pin["xq"], pin["xk"], pin["xv"], pin["conv_weight"], pin["a_raw"], pin["b_raw"],
                    decay_rate=pin["decay_rate"], gate_bias=pin["gate_bias"], conv_state=pin["conv_state"],
                    conv_state_out=pstate, outs=pouts)

    def prepare_decode():
        gdn.prepare(din["xq"], din["xk"], din["xv"], din["conv_weight"], din["a_raw"], din["b_raw"],
                    decay_rate=din["decay_rate"], gate_bias=din["gate_bias"], conv_state=din["conv_state"],
                    conv_state_out=din["conv_state"])

    # the 64K prefill from the raw projections in one pass: the preparation inside the chunk
    # kernels' loads
    fws = torch.empty(max(gdn.gdn_prepare_chunk_prefill_workspace_size(w.B, w.T, w.H, w.dk, w.dv, w.chunk, gdn.GDN_BF16),
                          1), device=dev, dtype=torch.uint8)

    def prepared_prefill():
        gdn.prepare_chunk_prefill(pin["xq"], pin["xk"], pin["xv"], pin["conv_weight"], pin["a_raw"], pin["b_raw"],
                                  pre["s0"], decay_rate=pin["decay_rate"], gate_bias=pin["gate_bias"],
                                  conv_state=pin["conv_state"], conv_state_out=pstate, chunk=w.chunk, out=out,
                                  final_state=fin, workspace=fws)

    # gradients of one prefill call on the training shape 1b_8k (B=4 H=32 T=8192 d=64)
    bw = gi.WORKLOADS[args.backward_workload]
    bin_ = gi.workload_inputs(args.backward_workload, device=dev)
    bdo = gi.draw_v((bw.B, bw.T, bw.H, bw.dv), gi.seed_of(bw.wid, 1, "v"), torch.float32, dev)
    f32 = dict(device=dev, dtype=torch.float32)
    bouts = (torch.empty((bw.B, bw.T, bw.H, bw.dk), **f32), torch.empty((bw.B, bw.T, bw.H, bw.dk), **f32),
             torch.empty((bw.B, bw.T, bw.H, bw.dv), **f32), torch.empty((bw.B, bw.T, bw.H), **f32),
             torch.empty((bw.B, bw.T, bw.H), **f32), torch.empty((bw.B, bw.H, bw.dk, bw.dv), **f32))
    bws = torch.empty(max(gdn.backward_workspace_bytes(bw.B, bw.T, bw.H, bw.dk, bw.dv, gdn.GDN_BF16), 1),
                      device=dev, dtype=torch.uint8)

    def backward():
        gdn.chunk_backward(bin_["q"], bin_["k"], bin_["v"], bin_["g"], bin_["beta"], bdo, None, None, outs=bouts,
                           workspace=bws)

    if args.only == "backward":
        for _ in range(args.warmup):
            backward()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            backward()
        torch.cuda.synchronize()
        print(json.dumps({"only": "backward", "steps": args.steps,
                          "wall_ms": (time.perf_counter() - t0) * 1e3}), flush=True)
        return

    if args.only == "prepare":
        # the preparation on both shapes, the prefill with the preparation in its loads, and the
        # one-launch decode step from the raw projections
        for _ in range(args.warmup):
            prepare()
            prepare_decode()
            prepared_prefill()
            decode_fused()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            prepare()
            prepare_decode()
            prepared_prefill()
            decode_fused()
        torch.cuda.synchronize()
        print(json.dumps({"only": "prepare", "steps": args.steps,
                          "wall_ms": (time.perf_counter() - t0) * 1e3}), flush=True)
        return

    def prefill():
        if args.only == "decode":
            return
        gdn.chunk_prefill(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["s0"],
                          chunk=w.chunk, out=out, final_state=fin, workspace=ws)

    def decode_chain(ev):
        if args.only == "prefill":
            return
        for s, d in enumerate(steps_in):
            ev[s][0].record(stream)
            gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=dout)
            ev[s][1].record(stream)

    mk = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        prefill()
        state.copy_(state0)
        decode_chain([(mk(), mk()) for _ in steps_in])
    torch.cuda.synchronize()

    pre_ev = [(mk(), mk()) for _ in range(args.steps)]
    dec_ev = [[(mk(), mk()) for _ in steps_in] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        pre_ev[i][0].record(stream)
        prefill()
        pre_ev[i][1].record(stream)
        state.copy_(state0)
        decode_chain(dec_ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    if args.only != "all":
        print(json.dumps({"only": args.only, "steps": args.steps, "wall_ms": wall * 1e3}), flush=True)
        return

    # the second rule (no erase term) on the same inputs, timed the same way; reported beside
    # the main figures, not part of `value`
    def decay_prefill():
        gdn.chunk_prefill(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["s0"], chunk=w.chunk,
                          out=out, final_state=fin, workspace=ws, rule=gdn.GDN_RULE_GATED_DECAY)
    for _ in range(args.warmup):
        decay_prefill()
    dp_ev = [(mk(), mk()) for _ in range(args.steps)]
    for a, b in dp_ev:
        a.record(stream)
        decay_prefill()
        b.record(stream)
    state.copy_(state0)
    dd_ev = [(mk(), mk()) for _ in steps_in]
    for s, d in enumerate(steps_in):
        dd_ev[s][0].record(stream)
        gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=dout,
                        rule=gdn.GDN_RULE_GATED_DECAY)
        dd_ev[s][1].record(stream)
    torch.cuda.synchronize()
    decay_pre_ms = sum(a.elapsed_time(b) for a, b in dp_ev) / len(dp_ev)
    decay_dec_ms = sum(a.elapsed_time(b) for a, b in dd_ev) / len(dd_ev)

    # packed variable-length prefill: 64 prompts of seeded lengths (1..2047 tokens, 74,178 in all)
    # into a 64-slot state pool, from zero states -- a continuous-batching prefill about the size
    # of the 64K call; reported beside the main figures
    import numpy as np
    lens = np.random.default_rng(11).integers(1, 2048, size=64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tv = int(cu[-1])
    vin = gi.prefill_inputs(1, Tv, w.H, w.dk, w.dv, wid=90, qkv_dtype=torch.bfloat16, device=dev)
    vin = {k: x[0] for k, x in vin.items() if x is not None}
    vpool = torch.zeros((64, w.H, w.dk, w.dv), device=dev, dtype=torch.float32)
    vout = torch.empty((Tv, w.H, w.dv), device=dev, dtype=torch.float32)
    vws = torch.empty(max(gdn.varlen_workspace_bytes(cu, w.H, w.dk, w.dv, w.chunk, gdn.GDN_BF16), 1),
                      device=dev, dtype=torch.uint8)
    no_init = np.zeros(64, dtype=np.int32)

    def varlen_prefill():
        gdn.chunk_prefill_varlen(vin["q"], vin["k"], vin["v"], vin["g"], vin["beta"], cu, vpool,
                                 has_initial=no_init, chunk=w.chunk, out=vout, workspace=vws)
    for _ in range(args.warmup):
        varlen_prefill()
    vl_ev = [(mk(), mk()) for _ in range(args.steps)]
    for a, b in vl_ev:
        a.record(stream)
        varlen_prefill()
        b.record(stream)
    torch.cuda.synchronize()
    varlen_ms = sum(a.elapsed_time(b) for a, b in vl_ev) / len(vl_ev)

    # the 1B-shaped 8K batch (B=4 H=32 T=8192 d=64, zero start state); reported beside the main figures
    w8 = gi.WORKLOADS["1b_8k"]
    p8 = gi.workload_inputs("1b_8k", device=dev)
    o8 = torch.empty((w8.B, w8.T, w8.H, w8.dv), device=dev, dtype=torch.float32)
    f8 = torch.empty((w8.B, w8.H, w8.dk, w8.dv), device=dev, dtype=torch.float32)
    ws8 = torch.empty(max(gdn.workspace_bytes(w8.B, w8.T, w8.H, w8.dk, w8.dv, w8.chunk, gdn.GDN_BF16), 1),
                      device=dev, dtype=torch.uint8)

    def prefill_8k():
        gdn.chunk_prefill(p8["q"], p8["k"], p8["v"], p8["g"], p8["beta"], None, chunk=w8.chunk, out=o8,
                          final_state=f8, workspace=ws8)
    for _ in range(args.warmup):
        prefill_8k()
    p8_ev = [(mk(), mk()) for _ in range(args.steps)]
    for a, b in p8_ev:
        a.record(stream)
        prefill_8k()
        b.record(stream)
    torch.cuda.synchronize()
    p8_ms = sorted(a.elapsed_time(b) for a, b in p8_ev)
    p8_avg = sum(p8_ms) / len(p8_ms)
    p8_th = w8.B * w8.T * w8.H
    p8_bytes = p8_th * BYTES_PER_TOKEN_HEAD + w8.B * w8.H * w8.dk * w8.dv * 4  # final state out; no start state
    del p8, o8, f8, ws8

    # one 64K call of the 3B-shaped chain (B=1 H=24 T=65536 d=128), state carried in and out;
    # reported beside the main figures
    w3 = gi.WORKLOADS["3b_2m"]
    p3 = gi.workload_inputs("3b_2m", call=1, device=dev)
    s3 = gi.draw_state((w3.B, w3.H, w3.dk, w3.dv), gi.seed_of(w3.wid, 1, "s0"), dev)
    o3 = torch.empty((w3.B, w3.T, w3.H, w3.dv), device=dev, dtype=torch.float32)
    f3 = torch.empty_like(s3)
    ws3 = torch.empty(max(gdn.workspace_bytes(w3.B, w3.T, w3.H, w3.dk, w3.dv, w3.chunk, gdn.GDN_BF16), 1),
                      device=dev, dtype=torch.uint8)

    def prefill_3b():
        gdn.chunk_prefill(p3["q"], p3["k"], p3["v"], p3["g"], p3["beta"], s3, chunk=w3.chunk, out=o3,
                          final_state=f3, workspace=ws3)
    for _ in range(args.warmup):
        prefill_3b()
    p3_ev = [(mk(), mk()) for _ in range(args.steps)]
    for a, b in p3_ev:
        a.record(stream)
        prefill_3b()
        b.record(stream)
    torch.cuda.synchronize()
    p3_ms = sum(a.elapsed_time(b) for a, b in p3_ev) / len(p3_ev)
    p3_th = w3.B * w3.T * w3.H
    p3_bytes = p3_th * BYTES_PER_TOKEN_HEAD_128 + 2 * w3.B * w3.H * w3.dk * w3.dv * 4
    del p3

    # the whole 3B-shaped 2M-token prefill: 32 chained 64K calls, each on its own inputs (all
    # resident before timing, 39 GB), the state carried from zeros through every call in place
    chain_in = [gi.workload_inputs("3b_2m", call=c, device=dev) for c in range(w3.calls)]
    s_chain = torch.zeros((w3.B, w3.H, w3.dk, w3.dv), device=dev, dtype=torch.float32)

    def chain_2m(ev=None):
        for c, d in enumerate(chain_in):
            if ev is not None:
                ev[c][0].record(stream)
            gdn.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], s_chain, chunk=w3.chunk, out=o3,
                              final_state=s_chain, workspace=ws3)
            if ev is not None:
                ev[c][1].record(stream)
    chain_2m()
    chain_ev, chain_call_ev = [], []
    for _ in range(3):
        s_chain.zero_()
        a, b = mk(), mk()
        calls_ev = [(mk(), mk()) for _ in chain_in]
        a.record(stream)
        chain_2m(calls_ev)
        b.record(stream)
        chain_ev.append((a, b))
        chain_call_ev += calls_ev
    torch.cuda.synchronize()
    chain_ms = sorted(a.elapsed_time(b) for a, b in chain_ev)
    chain_call_ms = sorted(a.elapsed_time(b) for a, b in chain_call_ev)
    chain_tokens = w3.B * w3.T * w3.calls
    del chain_in, s_chain, o3, ws3

    # preparation: alone (64K shape and decode batch), and followed by the 64K prefill
    for _ in range(args.warmup):
        prepare()
        prepare_decode()
        prepare_decode_pool()
        decode_fused()
        decode_separate()
    pp_ev = [(mk(), mk()) for _ in range(args.steps)]
    fu_ev = [(mk(), mk()) for _ in range(args.steps)]
    se_ev = [(mk(), mk()) for _ in range(args.steps)]
    pd_ev = [(mk(), mk()) for _ in range(args.steps)]
    pv_ev = [(mk(), mk()) for _ in range(args.steps)]
    pc_ev = [(mk(), mk()) for _ in range(args.steps)]
    for i in range(args.steps):
        pp_ev[i][0].record(stream)
        prepare()
        pp_ev[i][1].record(stream)
        pd_ev[i][0].record(stream)
        prepare_decode()
        pd_ev[i][1].record(stream)
        pv_ev[i][0].record(stream)
        prepare_decode_pool()
        pv_ev[i][1].record(stream)
        fu_ev[i][0].record(stream)
        decode_fused()
        fu_ev[i][1].record(stream)
        se_ev[i][0].record(stream)
        decode_separate()
        se_ev[i][1].record(stream)
    for i in range(args.steps):
        pc_ev[i][0].record(stream)
        prepare()
        gdn.chunk_prefill(pouts[0], pouts[1], pouts[2], pouts[3], pouts[4], pre["s0"], chunk=w.chunk,
                          out=out, final_state=fin, workspace=ws)
        pc_ev[i][1].record(stream)
    for _ in range(args.warmup):
        prepared_prefill()
    pf_ev = [(mk(), mk()) for _ in range(args.steps)]
    for a, b in pf_ev:
        a.record(stream)
        prepared_prefill()
        b.record(stream)
    torch.cuda.synchronize()
    fused_prefill_ms = sum(a.elapsed_time(b) for a, b in pf_ev) / len(pf_ev)
    del fws
    din["conv_state"].copy_(dstate0)
    prep_ms = sum(a.elapsed_time(b) for a, b in pp_ev) / len(pp_ev)
    prep_dec_ms = sum(a.elapsed_time(b) for a, b in pd_ev) / len(pd_ev)
    prep_pool_ms = sum(a.elapsed_time(b) for a, b in pv_ev) / len(pv_ev)
    prep_chain_ms = sum(a.elapsed_time(b) for a, b in pc_ev) / len(pc_ev)
    fused_ms = sum(a.elapsed_time(b) for a, b in fu_ev) / len(fu_ev)
    separate_ms = sum(a.elapsed_time(b) for a, b in se_ev) / len(se_ev)
    del fstate, fconv
    conv_ch = w.H * (2 * w.dk + w.dv)
    prep_bytes = w.B * w.T * w.H * PREP_BYTES_PER_TOKEN_HEAD + conv_ch * (16 + 24 * w.B)
    prep_dec_bytes = dw.B * dw.H * PREP_BYTES_PER_TOKEN_HEAD + conv_ch * (16 + 24 * dw.B)
    # fused step: raw q, k, v (bf16) + two logits in, the state read and written, o out, windows
    fused_bytes = (dw.B * dw.H * (3 * 64 * 2 + 2 * 4 + 2 * dw.dk * dw.dv * 4 + dw.dv * 4)
                   + conv_ch * (16 + 24 * dw.B))

    # backward on the training shape
    for _ in range(args.warmup):
        backward()
    bw_ev = [(mk(), mk()) for _ in range(max(2, args.steps // 2))]
    for a, b in bw_ev:
        a.record(stream)
        backward()
        b.record(stream)
    torch.cuda.synchronize()
    bwd_ms = sum(a.elapsed_time(b) for a, b in bw_ev) / len(bw_ev)
    bwd_flops = bw.B * bw.T * bw.H * BWD_FLOPS_PER_TOKEN_HEAD
    del bin_, bdo, bouts, bws

    # the gradients of a 3B-shaped layer's 8K training call (B=1 H=24 T=8192 d=128); reported
    # beside the main figures
    b3 = gi.prefill_inputs(1, 8192, 24, 128, 128, wid=244, device=dev)
    b3do = gi.draw_v((1, 8192, 24, 128), gi.seed_of(244, 1, "v"), torch.float32, dev)
    b3outs = (torch.empty((1, 8192, 24, 128), **f32), torch.empty((1, 8192, 24, 128), **f32),
              torch.empty((1, 8192, 24, 128), **f32), torch.empty((1, 8192, 24), **f32),
              torch.empty((1, 8192, 24), **f32), torch.empty((1, 24, 128, 128), **f32))
    b3ws = torch.empty(gdn.backward_workspace_bytes(1, 8192, 24, 128, 128, gdn.GDN_BF16), device=dev, dtype=torch.uint8)

    def backward_3b():
        gdn.chunk_backward(b3["q"], b3["k"], b3["v"], b3["g"], b3["beta"], b3do, None, None, outs=b3outs,
                           workspace=b3ws)
    for _ in range(args.warmup):
        backward_3b()
    b3_ev = [(mk(), mk()) for _ in range(max(2, args.steps // 4))]
    for a, b in b3_ev:
        a.record(stream)
        backward_3b()
        b.record(stream)
    torch.cuda.synchronize()
    bwd3_ms = sum(a.elapsed_time(b) for a, b in b3_ev) / len(b3_ev)
    del b3, b3do, b3outs, b3ws

    # decode on 3B-shaped states (256 sequences, H=24, 128 x 128 fp32 states, 402 MB): each state
    # takes four wavefronts of 32 key rows of whole 128-column rows; reported beside the main figures
    s128 = gi.decode_state(dw.B, 24, 128, 128, wid=95, device=dev)
    in128 = [gi.decode_inputs(dw.B, 24, 128, 128, t, wid=95, device=dev) for t in range(dw.calls)]
    o128 = torch.empty((dw.B, 24, 128), device=dev, dtype=torch.float32)
    for d in in128:
        gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s128, out=o128)
    d128_ev = [(mk(), mk()) for _ in range(max(3, args.steps // 2))]
    for a, b in d128_ev:
        a.record(stream)
        for d in in128:
            gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s128, out=o128)
        b.record(stream)
    torch.cuda.synchronize()
    d128_ms = sorted(a.elapsed_time(b) / len(in128) for a, b in d128_ev)
    d128_avg = sum(d128_ms) / len(d128_ms)
    d128_bytes = dw.B * 24 * (2 * 4 * 128 * 128 + 3 * 128 * 2 + 8 + 128 * 4)
    # the same states stepped from the raw projections, preparation and update in one launch
    f128 = gi.prep_inputs(dw.B, 1, 24, 128, 128, wid=203, device=dev)
    f128f = {kk: f128[kk][:, 0].contiguous() for kk in ("xq", "xk", "xv", "a_raw", "b_raw")}
    fconv128 = f128["conv_state"].clone()

    def decode_fused_128():
        gdn.prepare_decode_step(f128f["xq"], f128f["xk"], f128f["xv"], f128["conv_weight"], f128f["a_raw"],
                                f128f["b_raw"], fconv128, s128, decay_rate=f128["decay_rate"],
                                gate_bias=f128["gate_bias"], out=o128)
    for _ in range(args.warmup):
        decode_fused_128()
    f128_ev = [(mk(), mk()) for _ in range(args.steps)]
    for a, b in f128_ev:
        a.record(stream)
        decode_fused_128()
        b.record(stream)
    torch.cuda.synchronize()
    f128_ms = sum(a.elapsed_time(b) for a, b in f128_ev) / len(f128_ev)
    conv128 = 24 * 3 * 128
    f128_bytes = dw.B * 24 * (3 * 128 * 2 + 2 * 4 + 2 * 128 * 128 * 4 + 128 * 4) + conv128 * (16 + 24 * dw.B)
    del s128, in128, o128, f128, f128f, fconv128

    # decode over eight distinct states in rotation, one per GDN layer of an 8-GDN-layer hybrid: each
    # step updates layer 0's 128 MiB state, then layer 1's, ... (8 x 128 MiB = 1 GiB, four times the
    # 256 MB last-level cache), so every state read and every write-back of the previous layers'
    # dirty lines falls on DRAM inside the timed window; eager launches back to back, and the same
    # 8 x 16 launches replayed from one HIP graph
    n_layers = 8
    layer_states = [state0.clone() for _ in range(n_layers)]
    rot_launch = lambda: [gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st, out=dout)
                          for d in steps_in for st in layer_states]
    rot_launch()
    rot_ev = [(mk(), mk()) for _ in range(max(2, args.steps // 4))]
    for a, b in rot_ev:
        a.record(stream)
        rot_launch()
        b.record(stream)
    rot_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(rot_graph):
        rot_launch()
    rot_graph.replay()
    rotg_ev = [(mk(), mk()) for _ in range(max(2, args.steps // 4))]
    for a, b in rotg_ev:
        a.record(stream)
        rot_graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    n_rot = n_layers * len(steps_in)
    rot_us = sorted(a.elapsed_time(b) * 1e3 / n_rot for a, b in rot_ev)
    rotg_us = sorted(a.elapsed_time(b) * 1e3 / n_rot for a, b in rotg_ev)
    del layer_states, rot_graph

    # decode with a cold last-level cache: read a 1 GiB buffer before each step, outside the
    # events (a read leaves only clean lines behind, so no write-back competes with the step)
    flush = torch.ones(FLUSH_BYTES // 4, device=dev, dtype=torch.float32)
    sink = torch.empty((), device=dev, dtype=torch.float32)
    cold_ev = [[(mk(), mk()) for _ in steps_in] for _ in range(max(1, args.steps // 4))]
    for chain in cold_ev:
        state.copy_(state0)
        for s, d in enumerate(steps_in):
            torch.sum(flush, dim=0, out=sink)
            chain[s][0].record(stream)
            gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=dout)
            chain[s][1].record(stream)
    torch.cuda.synchronize()

    # the 16 decode steps captured once in a HIP graph and replayed, the way a serving loop
    # issues them: no host work between steps (the state is reset outside the graph)
    dec_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dec_graph):
        for d in steps_in:
            gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=dout)
    graph_ev = [(mk(), mk()) for _ in range(max(3, args.steps // 2))]
    for a, b in graph_ev:
        state.copy_(state0)
        a.record(stream)
        dec_graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    graph_ms = sorted(a.elapsed_time(b) / len(steps_in) for a, b in graph_ev)
    graph_avg = sum(graph_ms) / len(graph_ms)
    cold_ms = sorted(a.elapsed_time(b) for chain in cold_ev for a, b in chain)
    cold_avg = sum(cold_ms) / len(cold_ms)
    pre_ms = sorted(a.elapsed_time(b) for a, b in pre_ev)
    dec_ms = sorted(a.elapsed_time(b) for step in dec_ev for a, b in step)
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    med = lambda xs: xs[len(xs) // 2]

    token_heads = w.B * w.T * w.H
    state_bytes = 2 * w.B * w.H * w.dk * w.dv * 4  # start state in, final state out
    pre_bytes = token_heads * BYTES_PER_TOKEN_HEAD + state_bytes
    pre_flops = token_heads * FLOPS_PER_TOKEN_HEAD
    pre_gbps = pre_bytes / (pre_avg * 1e-3) / 1e9
    pre_tflops = pre_flops / (pre_avg * 1e-3) / 1e12
    tokens_per_s = w.B * w.T / (pre_avg * 1e-3)
    dec_bytes = dw.B * dw.H * DECODE_BYTES_PER_SEQ_HEAD
    dec_gbps = dec_bytes / (dec_avg * 1e-3) / 1e9
    cold_gbps = dec_bytes / (cold_avg * 1e-3) / 1e9

    result = {
        "metric": "GDN prefill tokens/s at 64K (% bf16 MFMA peak); decode GB/s (% HBM peak)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "1b_64k prefill: B=1 H=32 T=65536 d_k=d_v=64 chunk=64, bf16 q/k/v, fp32 g/beta/state, "
                        "start state carried in; plus decode: N=256 H=32 d=64, 16 steps",
            "B": w.B, "H": w.H, "T": w.T, "d_k": w.dk, "d_v": w.dv, "chunk": w.chunk,
            "decode_sequences": dw.B, "decode_steps": dw.calls,
        },
        "prefill": {
            "ms_avg": round(pre_avg, 4), "ms_median": round(med(pre_ms), 4), "ms_min": round(pre_ms[0], 4),
            "GBps_algorithmic": round(pre_gbps, 1), "hbm_frac": round(pre_gbps / HBM_PEAK_GBPS, 4),
            "useful_TFLOPs": round(pre_tflops, 2), "mfma_frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
            "ceiling_mfma_frac": round(CEILING_MFMA_FRAC, 4),
            "frac_of_ceiling": round(pre_tflops / BF16_PEAK_TFLOPS / CEILING_MFMA_FRAC, 4),
            "bytes_per_call": pre_bytes, "useful_flops_per_call": pre_flops,
            "note": "ceiling_mfma_frac: the useful-MFMA fraction the HBM floor allows (algorithmic bytes at 8 TB/s), "
                    "frac_of_ceiling: mfma_frac over it (= hbm_frac); the kernels run the chunk form in 32-token "
                    "chunks (chunk=64 is the longest the call allows)",
        },
        "decode": {
            "us_per_step_avg": round(dec_avg * 1e3, 2), "us_per_step_median": round(med(dec_ms) * 1e3, 2),
            "GBps": round(dec_gbps, 1), "hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
            "bytes_per_step": dec_bytes,
            "cold_us_per_step_avg": round(cold_avg * 1e3, 2), "cold_GBps": round(cold_gbps, 1),
            "cold_hbm_frac": round(cold_gbps / HBM_PEAK_GBPS, 4),
            "graph_us_per_step_avg": round(graph_avg * 1e3, 2),
            "graph_GBps": round(dec_bytes / (graph_avg * 1e-3) / 1e9, 1),
            "graph_hbm_frac": round(dec_bytes / (graph_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic_bytes_per_step": recorded_traffic("decode"),
            "dram_bound_hbm_frac": round(dec_bytes / (sum(rot_us) / len(rot_us) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "warm: 16 back-to-back steps launched from Python, each between its own events (host "
                    "launch gaps included), the 128 MiB state can stay in the 256 MB last-level cache; cold: a "
                    "1 GiB buffer is read before every step; graph: the 16 steps replayed from one HIP graph, "
                    "time / 16; dram_bound_hbm_frac: the headline decode figure, the same step over eight "
                    "distinct states in rotation (decode_8_layers), every state access from DRAM",
        },
        "decode_8_layers": {
            "workload": "the 256 x 32 x 64 decode step over 8 distinct 128 MiB states in rotation (one per GDN "
                        "layer; 1 GiB of states, 4x the last-level cache), 16 steps x 8 layers",
            "us_per_layer_step_avg": round(sum(rot_us) / len(rot_us), 2),
            "GBps": round(dec_bytes / (sum(rot_us) / len(rot_us) * 1e-6) / 1e9, 1),
            "hbm_frac": round(dec_bytes / (sum(rot_us) / len(rot_us) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "graph_us_per_layer_step_avg": round(sum(rotg_us) / len(rotg_us), 2),
            "graph_GBps": round(dec_bytes / (sum(rotg_us) / len(rotg_us) * 1e-6) / 1e9, 1),
            "graph_hbm_frac": round(dec_bytes / (sum(rotg_us) / len(rotg_us) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        },
        "decode_3b_shape": {
            "workload": "256 sequences, H=24, d_k=d_v=128 fp32 states (402 MB), 16 steps launched back to back",
            "us_per_step_avg": round(d128_avg * 1e3, 2), "bytes_per_step": d128_bytes,
            "GBps": round(d128_bytes / (d128_avg * 1e-3) / 1e9, 1),
            "hbm_frac": round(d128_bytes / (d128_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "fused_step_us_avg": round(f128_ms * 1e3, 2), "fused_step_bytes": f128_bytes,
            "fused_step_hbm_frac": round(f128_bytes / (f128_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "fused_step: gdn_prepare_decode_step on the same states, the preparation from raw bf16 "
                    "projections and the state update in one launch",
        },
        "varlen_prefill": {
            "sequences": 64, "tokens": Tv, "ms_avg": round(varlen_ms, 4),
            "tokens_per_s": round(Tv / (varlen_ms * 1e-3), 1),
            "GBps_algorithmic": round(Tv * w.H * BYTES_PER_TOKEN_HEAD / (varlen_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(Tv * w.H * BYTES_PER_TOKEN_HEAD / (varlen_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "64 packed prompts of seeded lengths 1..2047, H=32 d=64 chunk 64, zero start states "
                    "written to a 64-slot pool",
        },
        "prepare": {
            "ms_avg": round(prep_ms, 4), "GBps_algorithmic": round(prep_bytes / (prep_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(prep_bytes / (prep_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_call": prep_bytes,
            "decode_us_avg": round(prep_dec_ms * 1e3, 2),
            "decode_GBps_algorithmic": round(prep_dec_bytes / (prep_dec_ms * 1e-3) / 1e9, 1),
            "decode_pool_us_avg": round(prep_pool_ms * 1e3, 2),
            "decode_step_fused_us_avg": round(fused_ms * 1e3, 2),
            "decode_step_fused_hbm_frac": round(fused_bytes / (fused_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "decode_step_separate_us_avg": round(separate_ms * 1e3, 2),
            "decode_step_fused_traffic_bytes": recorded_traffic("fused"),
            "traffic_bytes_per_call": recorded_traffic("prepare"),
            "prepare_then_prefill_ms_avg": round(prep_chain_ms, 4),
            "prepare_then_prefill_tokens_per_s": round(w.B * w.T / (prep_chain_ms * 1e-3), 1),
            "prepared_prefill_ms_avg": round(fused_prefill_ms, 4),
            "prepared_prefill_tokens_per_s": round(w.B * w.T / (fused_prefill_ms * 1e-3), 1),
            "prepared_prefill_traffic_bytes": recorded_traffic("prepared"),
            "note": "short causal convolution + SiLU + q/k L2 norm + gate activations on the 64K shape "
                    "(bf16 in and out) and on the 256-sequence decode batch (state in place; decode_pool: the "
                    "same step as 256 one-token packed sequences with states in a 512-slot pool; decode_step_fused: "
                    "preparation and state update of that batch in one launch, decode_step_separate: the same as "
                    "gdn_prepare + gdn_decode_step; prepared_prefill: gdn_prepare_chunk_prefill, the preparation done "
                    "in the prefill kernels' loads, against prepare_then_prefill, the two calls)",
        },
        "backward": {
            "workload": "1b_8k: B=4 H=32 T=8192 d_k=d_v=64, bf16 q/k/v, gated delta rule, zero start state",
            "ms_avg": round(bwd_ms, 4), "tokens_per_s": round(bw.B * bw.T / (bwd_ms * 1e-3), 1),
            "TFLOPs_fp32": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
            "alu_frac": round(bwd_flops / (bwd_ms * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS, 4),
            "flops_per_call": bwd_flops,
            "note": "forward recompute (keeps chunk start states) + per-chunk maps + reverse scan + per-chunk "
                    "gradients; products as three-pass hi/lo bf16 MFMA (fp32-class results) except the gate "
                    "prefix sums and the 16x16 inverse blocks (fp32 MFMA); FLOPs are the gradient "
                    "kernels' useful multiply-adds x 2, alu_frac against the fp32 peak (the precision delivered)",
        },
        "backward_3b_shape": {
            "workload": "one 3B-shaped layer's 8K training call: B=1 H=24 T=8192 d_k=d_v=128, bf16 q/k/v, gated "
                        "delta rule, zero start state",
            "ms_avg": round(bwd3_ms, 4), "tokens_per_s": round(8192 / (bwd3_ms * 1e-3), 1),
            "note": "the gradient pass keeps its larger matrices in global scratch (they do not fit on chip)",
        },
        "prefill_1b_8k": {
            "workload": "1b_8k: B=4 H=32 T=8192 d_k=d_v=64 chunk 64, bf16 q/k/v, zero start state, final state out",
            "ms_avg": round(p8_avg, 4), "ms_median": round(p8_ms[len(p8_ms) // 2], 4),
            "tokens_per_s": round(w8.B * w8.T / (p8_avg * 1e-3), 1),
            "GBps_algorithmic": round(p8_bytes / (p8_avg * 1e-3) / 1e9, 1),
            "hbm_frac": round(p8_bytes / (p8_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "useful_TFLOPs": round(p8_th * FLOPS_PER_TOKEN_HEAD / (p8_avg * 1e-3) / 1e12, 2),
        },
        "prefill_3b_64k": {
            "workload": "one 64K call of the 3B-shaped chain: B=1 H=24 T=65536 d_k=d_v=128 chunk 64, bf16 q/k/v, "
                        "state carried in and out",
            "ms_avg": round(p3_ms, 4), "tokens_per_s": round(w3.B * w3.T / (p3_ms * 1e-3), 1),
            "GBps_algorithmic": round(p3_bytes / (p3_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(p3_bytes / (p3_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "useful_TFLOPs": round(p3_th * FLOPS_PER_TOKEN_HEAD_128 / (p3_ms * 1e-3) / 1e12, 2),
        },
        "prefill_3b_2m_chain": {
            "workload": "3B-shaped 2M-token prefill: 32 chained calls of B=1 H=24 T=65536 d_k=d_v=128 chunk 64, "
                        "each on its own inputs, state carried from zeros through every call in place",
            "calls": w3.calls, "tokens": chain_tokens,
            "ms_median": round(chain_ms[len(chain_ms) // 2], 3), "ms_min": round(chain_ms[0], 3),
            "ms_per_call_median": round(chain_call_ms[len(chain_call_ms) // 2], 4),
            "tokens_per_s": round(chain_tokens / (chain_ms[len(chain_ms) // 2] * 1e-3), 1),
            "GBps_algorithmic": round((chain_tokens * w3.H * BYTES_PER_TOKEN_HEAD_128
                                       + w3.calls * 2 * w3.B * w3.H * w3.dk * w3.dv * 4)
                                      / (chain_ms[len(chain_ms) // 2] * 1e-3) / 1e9, 1),
        },
        "gated_decay_rule": {
            "prefill_ms_avg": round(decay_pre_ms, 4),
            "prefill_tokens_per_s": round(w.B * w.T / (decay_pre_ms * 1e-3), 1),
            "prefill_GBps_algorithmic": round(pre_bytes / (decay_pre_ms * 1e-3) / 1e9, 1),
            "prefill_hbm_frac": round(pre_bytes / (decay_pre_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "decode_us_per_step_avg": round(decay_dec_ms * 1e3, 2),
            "decode_GBps": round(dec_bytes / (decay_dec_ms * 1e-3) / 1e9, 1),
            "decode_hbm_frac": round(dec_bytes / (decay_dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "S_t = a_t S_{t-1} + b_t v_t k_t^T (no erase term) on the same 64K and decode inputs",
        },
        "roofline": {
            "kernel": "one gdn_chunk_prefill call: chunk_kernel MAP + chain_kernel + chunk_kernel OUT",
            "bound": "hbm", "achieved": round(pre_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(pre_gbps / HBM_PEAK_GBPS, 4), "traffic": recorded_traffic("prefill"),
        },
    }

    if not args.no_cpu_baseline:
        import oracle  # test infrastructure: timed here as the reported CPU baseline only
        T = min(args.cpu_tokens, w.T)
        sl = {k: (None if k == "s0" else pre[k][:, :T].cpu()) for k in ("q", "k", "v", "g", "beta")}
        s0 = pre["s0"].cpu()
        t1 = time.perf_counter()
        oracle.prefill(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], s0)
        cpu_s = time.perf_counter() - t1
        cores = oracle.num_threads()
        # the same on one thread and one head, so the scaling over the host cores is visible
        one = {k: x[:, :, :1].contiguous() for k, x in sl.items()}
        oracle.set_num_threads(1)
        t1 = time.perf_counter()
        oracle.prefill(one["q"], one["k"], one["v"], one["g"], one["beta"], s0[:, :1].contiguous())
        one_s = time.perf_counter() - t1
        oracle.set_num_threads(cores)
        result["cpu_baseline"] = {
            "value": round(w.B * T / cpu_s, 1), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fp64 token-by-token oracle on the first {T} tokens of the 1b_64k workload, "
                      f"all {w.H} heads and value rows ({cpu_s:.2f} s)",
            "token_heads_per_s": round(w.B * T * w.H / cpu_s, 1),
            "single_thread_token_heads_per_s": round(w.B * T / one_s, 1),
            "single_thread_sample": f"one head of the same tokens on one thread ({one_s:.2f} s)",
        }

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
