#!/usr/bin/env python3
"""Benchmark of the GDN mixer hot path on one MI355X.

Prefill (the headline `value`): one step is the whole prefill mixer over one
synthetic batch of the hybrid model's GDN shape -- B=1, T=4096, 16 q/k heads,
32 v heads, d=128, chunk 64, bf16: gdn_conv1d_fwd (width-4 conv + SiLU) then
gdn_chunk_fwd (chunked gated delta rule, fp32 state) with the fused gated
RMSNorm epilogue writing bf16.  value = tokens/s.

Decode (reported beside it): one step is the decode mixer for 64 requests,
one token each -- gdn_conv1d_fwd in decode mode then gdn_recurrent_step with
the fused norm -- on per-request fp32 states of 32 x 128 x 128; reported as
state GB/s (2 x state bytes per step) and steps/s, and the same step through
gdn_mixer_decode_step, which does the conv, the recurrence and the norm in one
launch (bit-identical results).

Fused gates (reported beside them): the chunk and decode calls again through
gdn_chunk_fwd_gated / gdn_recurrent_step_gated, which form g and beta in their
prologues from bf16 raw gate projections (a packed b|a tensor) and per-head
a_log, as a model's B/A projections deliver them.

Both legs rotate over `--sets` independent copies of their buffers (as the
GDN layers of a model would), so the working set exceeds the 256 MB Infinity
Cache and the numbers are HBM-cold.  Inputs are resident in HBM before the
timed region starts.  Timing: W warmup steps, then K steps bracketed by
torch.cuda.synchronize() and HIP events on the stream the kernels run on.

Roofline of the dominant entry point gdn_chunk_fwd (prep + scan kernels):
algorithmic flops of the chunked method, 139,648 per token per v-head
(4.469 MFLOP per token), over its event-timed average duration, against the
dense bf16 matrix-core peak.  The CPU baseline times the float64 oracle on a
bounded sample on the host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
FLOP_PER_TOKEN_HEAD = 139_648  # chunked gated delta rule, C=64, d=128 (algorithmic)

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# on this workload (FETCH scaled by 2.0 and WRITE by 1.0, the readings of a
# 256 MiB device-to-device copy; see profiles/), valid for the kernel sources
# with these hashes (sha256, first 16 hex digits).  A kernel changed since the
# counters were taken reports null.
CSRC = os.path.join(ROOT, "gated_deltanet_mixer_causal_amd", "csrc")
CHUNK_SOURCES = {"chunk.hip": "34a28395d94d9929", "chunk_impl.hpp": "00117838d6369ddb",
                 "common.hpp": "48a2a30823c83686", "launch.hpp": "3c7351067da3f401"}
MEASURED_TRAFFIC = {
    "gdn_chunk_fwd": (289_238_630, CHUNK_SOURCES),
    "gdn_recurrent_step": (274_533_171, {"recurrent.hip": "feb115db1f28a22c", "common.hpp": "48a2a30823c83686",
                                         "launch.hpp": "3c7351067da3f401"}),
}


def measured_traffic(entry):
    import hashlib
    nbytes, sources = MEASURED_TRAFFIC[entry]
    for name, digest in sources.items():
        with open(os.path.join(CSRC, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != digest:
                return None
    return nbytes


# Executed matrix-core work per gdn_chunk_fwd launch on the same workload, from
# rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 and SQ_INSTS_VALU_MFMA_MOPS_F32
# (512 FLOP per op) summed over the prep and scan kernels; hash-gated like the
# traffic above.
MEASURED_MFMA = {
    "gdn_chunk_fwd": ((2_621_440 + 69_206_016) * 512, 524_288 * 512, CHUNK_SOURCES),
}


def measured_mfma(entry):
    bf16, f32, sources = MEASURED_MFMA[entry]
    if bf16 is None:
        return None
    import hashlib
    for name, digest in sources.items():
        with open(os.path.join(CSRC, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != digest:
                return None
    return bf16, f32


def call_stats(fn, n, start, torch):
    """Per-call durations (ms) of n calls fn(start + i), each between its own events."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fn(start + i)
        b.record(stream)
    torch.cuda.synchronize()
    import statistics
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return {"n": n, "median_ms": round(statistics.median(t), 4), "min_ms": round(t[0], 4),
            "max_ms": round(t[-1], 4), "std_ms": round(statistics.pstdev(t), 4)}


def environment(torch):
    props = torch.cuda.get_device_properties(0)
    return {"rocm_hip": torch.version.hip, "arch": getattr(props, "gcnArchName", None)}


def streaming_probes(torch):
    """What plain streaming kernels of the library reach on this GPU, per traffic shape (GB/s over the
    bytes each moves), on buffers rotated so no pass finds its data in the 256 MB Infinity Cache."""
    dev = "cuda:0"
    n = 32 << 20                                    # 128 MiB of fp32
    bufs = [torch.ones(n, device=dev) for _ in range(12)]

    def rate(fn, nbytes, reps=20):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return round(nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)

    def fill(i):                                    # write 512 MiB
        for j in range(4):
            bufs[(4 * i + j) % 12].fill_(float(i))

    def copy(i):                                    # read 128 MiB, write 128 MiB
        bufs[(2 * i) % 12].copy_(bufs[(2 * i + 7) % 12])

    def fan4(i):                                    # read 128 MiB once, write it four times
        src = bufs[(5 * i) % 12]
        for j in range(4):
            bufs[(5 * i + 1 + j) % 12].copy_(src)

    out = {"fill_512MiB_GB_per_s": rate(fill, 4 * n * 4), "copy_128MiB_GB_per_s": rate(copy, 2 * n * 4),
           "read_once_write_4x_GB_per_s": rate(fan4, 8 * n * 4),
           "note": "torch fill_ / copy_ kernels; the fan-out re-reads its source from cache for the last three "
                   "copies, so it counts 4 reads + 4 writes"}
    del bufs
    return out


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4, help="independent buffer sets rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the gdn_chunk_bwd timing")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the varlen (8 packed sequences) and long-context (16 x 8192 + 256 decode) legs")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the speculative-verification and mixed prefill-plus-decode timings")
    ap.add_argument("--copy-probe", action="store_true",
                    help="before the timed legs, copy 256 MiB device-to-device once (a plain copy of known "
                         "size that calibrates the FETCH_SIZE / WRITE_SIZE counters), then time plain streaming "
                         "kernels of the library (fill, copy, one read fanned out to four writes) and report them")
    return ap.parse_args()


def timed(fn, steps, warmup, torch):
    """Run fn(i) warmup times, then `steps` times between events; returns ms per step."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fn(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return e0.elapsed_time(e1) / steps, wall


def prefill_leg(args, torch, np, ops, I):
    lay = I.MODEL_LAYOUT
    d = I.model_prefill_inputs()
    T = d["x"].shape[0]
    dev = "cuda:0"

    def up(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).to(dev)

    ws_bytes = ops.gdn_chunk_fwd_workspace_size(lay.h_qk, lay.h_v, lay.d_k, lay.d_v, lay.chunk, 1, T,
                                                torch.bfloat16, True)
    sets = []
    x0 = up(d["x"], torch.bfloat16)
    gt = I.raw_gate_inputs(11, T, lay.h_v, dtype="bf16")
    ba0 = up(np.concatenate([gt["b"], gt["a"]], axis=1), torch.bfloat16)
    a_log = up(gt["a_log"])
    for _ in range(args.sets):
        s = dict(x=x0.clone(), w=up(d["conv_w"], torch.bfloat16), tail=up(d["tail"], torch.bfloat16),
                 cu=torch.from_numpy(d["cu_seqlens"]).to(dev), g=up(d["g"]), beta=up(d["beta"]),
                 z=up(d["z"], torch.bfloat16), nw=up(d["norm_w"]),
                 state=torch.zeros((1, lay.h_v, lay.d_v, lay.d_k), device=dev),
                 y_conv=torch.empty((T, lay.channels), dtype=torch.bfloat16, device=dev),
                 y=torch.empty((T, lay.h_v, lay.d_v), dtype=torch.bfloat16, device=dev),
                 o=torch.empty((T, lay.h_v, lay.d_v), dtype=torch.bfloat16, device=dev),
                 ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev))
        s["q"], s["k"], s["v"] = ops.qkv_views(s["y_conv"], lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
        s["ba"] = ba0.clone()
        s["a"], s["b"] = s["ba"][:, lay.h_v:], s["ba"][:, :lay.h_v]
        sets.append(s)
    del x0, ba0

    def step(i):
        s = sets[i % len(sets)]
        ops.gdn_conv1d_fwd(s["x"], s["w"], s["tail"], s["y_conv"], cu_seqlens=s["cu"])
        ops.gdn_chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["y"], chunk=lay.chunk, cu_seqlens=s["cu"],
                          initial_state=None, final_state=s["state"], z=s["z"], norm_w=s["nw"],
                          workspace=s["ws"])

    def chunk_only(i):
        s = sets[i % len(sets)]
        ops.gdn_chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["o"], chunk=lay.chunk, cu_seqlens=s["cu"],
                          final_state=s["state"], workspace=s["ws"])

    def chunk_gated(i):
        s = sets[i % len(sets)]
        ops.gdn_chunk_fwd_gated(s["q"], s["k"], s["v"], s["a"], s["b"], a_log, s["o"], chunk=lay.chunk,
                                cu_seqlens=s["cu"], final_state=s["state"], workspace=s["ws"])

    ms, wall = timed(step, args.steps, args.warmup, torch)
    ms_chunk, _ = timed(chunk_only, args.steps, args.warmup, torch)
    stats = call_stats(chunk_only, max(args.steps, 50), args.warmup + args.steps, torch)
    ms_chunk_gated, _ = timed(chunk_gated, args.steps, args.warmup, torch)
    ms_bwd = ms_conv_bwd = None
    if not args.no_backward:
        # gradients of the same call: d_o for every output, a final-state gradient
        bw = dict(do=torch.randn((T, lay.h_v, lay.d_v), device=dev),
                  dfin=torch.randn((1, lay.h_v, lay.d_v, lay.d_k), device=dev),
                  dq=torch.empty((T, lay.h_qk, lay.d_k), device=dev), dk=torch.empty((T, lay.h_qk, lay.d_k), device=dev),
                  dv=torch.empty((T, lay.h_v, lay.d_v), device=dev), dg=torch.empty((T, lay.h_v), device=dev),
                  dbeta=torch.empty((T, lay.h_v), device=dev),
                  dinit=torch.empty((1, lay.h_v, lay.d_v, lay.d_k), device=dev),
                  ws=torch.empty(ops.gdn_chunk_bwd_workspace_size(lay.h_qk, lay.h_v, lay.d_k, lay.d_v, 1, T),
                                 dtype=torch.uint8, device=dev))

        def backward(i):
            s = sets[i % len(sets)]
            ops.gdn_chunk_bwd(s["q"], s["k"], s["v"], s["g"], s["beta"], bw["do"], bw["dq"], bw["dk"], bw["dv"],
                              bw["dg"], bw["dbeta"], cu_seqlens=s["cu"], d_final=bw["dfin"], d_initial=bw["dinit"],
                              workspace=bw["ws"])

        ms_bwd, _ = timed(backward, max(2, args.steps // 4), 1, torch)
        del bw
        cb = dict(dy=torch.randn((T, lay.channels), device=dev), dx=torch.empty((T, lay.channels), device=dev),
                  dw=torch.empty((lay.channels, 4), device=dev),
                  dhi=torch.empty((1, 3, lay.channels), device=dev))

        def conv_backward(i):
            s = sets[i % len(sets)]
            ops.gdn_conv1d_bwd(s["x"], s["w"], cb["dy"], cb["dx"], cb["dw"], cu_seqlens=s["cu"],
                               conv_state_in=s["tail"], d_state_in=cb["dhi"])

        ms_conv_bwd, _ = timed(conv_backward, args.steps, args.warmup, torch)
        del cb
    return dict(T=T, ms=ms, wall=wall, ms_chunk=ms_chunk, chunk_stats=stats, layout=lay,
                ms_chunk_gated=ms_chunk_gated, ms_bwd=ms_bwd, ms_conv_bwd=ms_conv_bwd)


def decode_leg(args, torch, np, ops, I):
    lay = I.MODEL_LAYOUT
    n_req = 64
    dev = "cuda:0"
    d = I.decode_inputs(2, lay, n_req, 8)

    def up(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).to(dev)

    state0 = up(d["state"])
    sets = []
    for _ in range(args.sets):
        s = dict(state=state0.clone(), tail=up(d["tail"], torch.bfloat16), w=up(d["conv_w"], torch.bfloat16),
                 nw=up(d["norm_w"]), y_conv=torch.empty((n_req, lay.channels), dtype=torch.bfloat16, device=dev),
                 o=torch.empty((n_req, lay.h_v, lay.d_v), dtype=torch.bfloat16, device=dev))
        s["q"], s["k"], s["v"] = ops.qkv_views(s["y_conv"], lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
        sets.append(s)
    del state0
    steps_in = [dict(x=up(d["x"][t], torch.bfloat16), g=up(d["g"][t]), beta=up(d["beta"][t]),
                     z=up(d["z"][t], torch.bfloat16)) for t in range(d["x"].shape[0])]
    gate_in = []
    for t in range(d["x"].shape[0]):
        gt = I.raw_gate_inputs(20 + t, n_req, lay.h_v, dtype="bf16")
        ba = up(np.concatenate([gt["b"], gt["a"]], axis=1), torch.bfloat16)
        gate_in.append(dict(a=ba[:, lay.h_v:], b=ba[:, :lay.h_v], a_log=up(gt["a_log"])))

    def step(i):
        s = sets[i % len(sets)]
        inp = steps_in[i % len(steps_in)]
        ops.gdn_conv1d_fwd(inp["x"], s["w"], s["tail"], s["y_conv"])
        ops.gdn_recurrent_step(s["q"], s["k"], s["v"], inp["g"], inp["beta"], s["state"], s["o"], z=inp["z"],
                               norm_w=s["nw"])

    def fused_step(i):
        s = sets[i % len(sets)]
        inp = steps_in[i % len(steps_in)]
        ops.gdn_mixer_decode_step(inp["x"], s["w"], s["tail"], inp["g"], inp["beta"], s["state"], s["o"],
                                  h_qk=lay.h_qk, z=inp["z"], norm_w=s["nw"])

    def rec_only(i):
        s = sets[i % len(sets)]
        inp = steps_in[i % len(steps_in)]
        ops.gdn_recurrent_step(s["q"], s["k"], s["v"], inp["g"], inp["beta"], s["state"], s["o"])

    def rec_gated(i):
        s = sets[i % len(sets)]
        gi = gate_in[i % len(gate_in)]
        ops.gdn_recurrent_step_gated(s["q"], s["k"], s["v"], gi["a"], gi["b"], gi["a_log"], s["state"], s["o"])

    ms, wall = timed(step, args.steps, args.warmup, torch)
    ms_fused, _ = timed(fused_step, args.steps, args.warmup, torch)
    ms_rec, _ = timed(rec_only, args.steps, args.warmup, torch)
    rec_stats = call_stats(rec_only, max(args.steps, 50), args.warmup + args.steps, torch)
    ms_rec_gated, _ = timed(rec_gated, args.steps, args.warmup, torch)

    def rec_warm(i):   # one buffer set: its 128 MiB of state can stay in the 256 MB Infinity Cache
        s = sets[0]
        inp = steps_in[i % len(steps_in)]
        ops.gdn_recurrent_step(s["q"], s["k"], s["v"], inp["g"], inp["beta"], s["state"], s["o"])

    ms_rec_warm, _ = timed(rec_warm, args.steps, args.warmup, torch)
    state_bytes = n_req * lay.h_v * lay.d_v * lay.d_k * 4
    # per request: q, k, v, z (bf16), g, beta (fp32), o (bf16)
    small = n_req * (2 * lay.h_qk * lay.d_k * 2 + lay.h_v * lay.d_v * 2 + 2 * lay.h_v * 4 + lay.h_v * lay.d_v * 2)
    return dict(ms=ms, wall=wall, ms_rec=ms_rec, rec_stats=rec_stats, n_req=n_req, state_bytes=state_bytes,
                small=small, ms_rec_gated=ms_rec_gated, ms_rec_warm=ms_rec_warm, ms_fused=ms_fused)


def serving_leg(args, torch, np, ops, I):
    """Speculative verification (64 requests x 4 draft tokens, eight checkpoint
    columns per request, then restoring an accepted prefix) and one mixed
    prefill-plus-decode batch (four 1024-token prompt chunks, two of them fresh,
    and 60 decode tokens over pools of 128 slots), both with the fused norm and
    bf16 outputs, on one buffer set."""
    lay = I.MODEL_LAYOUT
    dev = "cuda:0"

    def up(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).to(dev)

    n_req, w_tok, n_cols = 64, 4, 8
    d = I.decode_inputs(5, lay, n_req, w_tok)
    rows = n_req * w_tok
    # request r's tokens are rows r * W .. r * W + W - 1
    x = up(d["x"].transpose(1, 0, 2).reshape(rows, -1), torch.bfloat16)
    g = up(d["g"].transpose(1, 0, 2).reshape(rows, -1))
    beta = up(d["beta"].transpose(1, 0, 2).reshape(rows, -1))
    z = up(d["z"].transpose(1, 0, 2, 3).reshape(rows, lay.h_v, lay.d_v), torch.bfloat16)
    state = up(d["state"])
    tail = up(d["tail"], torch.bfloat16)
    w = up(d["conv_w"], torch.bfloat16)
    nw = up(d["norm_w"])
    ckpt = torch.empty((n_req, n_cols) + tuple(state.shape[1:]), device=dev)
    win = torch.empty((n_req, n_cols, 3, lay.channels), dtype=torch.bfloat16, device=dev)
    y_conv = torch.empty((rows, lay.channels), dtype=torch.bfloat16, device=dev)
    o = torch.empty((rows, lay.h_v, lay.d_v), dtype=torch.bfloat16, device=dev)
    q, k, v = ops.qkv_views(y_conv, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    live = torch.arange(n_req, dtype=torch.int32, device=dev)
    accepted = (live * n_cols + 1).to(torch.int32)   # column 1: two of the four tokens accepted
    ckpt_rows = ckpt.view(n_req * n_cols, *state.shape[1:])

    def verify(i):
        ops.gdn_conv1d_verify(x, w, tail, y_conv, win, n_tok=w_tok)
        ops.gdn_recurrent_verify(q, k, v, g, beta, state, ckpt, o, n_tok=w_tok, z=z, norm_w=nw)

    def rec_verify(i):
        ops.gdn_recurrent_verify(q, k, v, g, beta, state, ckpt, o, n_tok=w_tok, z=z, norm_w=nw)

    def restore(i):
        ops.gdn_state_rows_copy(state, live, ckpt_rows, accepted)

    ms_verify, _ = timed(verify, args.steps, args.warmup, torch)
    ms_rec_verify, _ = timed(rec_verify, args.steps, args.warmup, torch)
    ms_restore, _ = timed(restore, args.steps, args.warmup, torch)
    del ckpt, win, d

    # mixed batch: sequences 0-3 prompt chunks (0 and 2 fresh), 4-63 single decode tokens
    lengths = [1024] * 4 + [1] * 60
    n_slots = 128
    m = I.mixed_batch_inputs(6, lay, lengths, n_slots)
    slots = np.random.default_rng(7).permutation(n_slots)[:len(lengths)].astype(np.int32)
    fresh = np.zeros(len(lengths), np.int32)
    fresh[[0, 2]] = 1
    t_cap = m["t_cap"]
    mx = up(m["x"], torch.bfloat16)
    mw = up(m["conv_w"], torch.bfloat16)
    mtail = up(m["tail_pool"], torch.bfloat16)
    mstate = up(m["state_pool"])
    cu = torch.from_numpy(m["cu_seqlens"]).to(dev)
    sl, fr = torch.from_numpy(slots).to(dev), torch.from_numpy(fresh).to(dev)
    mg, mb = up(m["g"]), up(m["beta"])
    mz, mnw = up(m["z"], torch.bfloat16), up(m["norm_w"])
    my_conv = torch.empty((t_cap, lay.channels), dtype=torch.bfloat16, device=dev)
    mq, mk, mv = ops.qkv_views(my_conv, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    my = torch.empty((t_cap, lay.h_v, lay.d_v), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(ops.gdn_chunk_fwd_workspace_size(lay.h_qk, lay.h_v, lay.d_k, lay.d_v, lay.chunk, len(lengths),
                                                      t_cap, torch.bfloat16, True), dtype=torch.uint8, device=dev)

    def mixed(i):
        ops.gdn_conv1d_mixed(mx, mw, mtail, my_conv, cu_seqlens=cu, state_slots=sl, fresh=fr)
        ops.gdn_chunk_mixed(mq, mk, mv, mg, mb, mstate, my, chunk=lay.chunk, cu_seqlens=cu, state_slots=sl,
                            fresh=fr, z=mz, norm_w=mnw, workspace=ws)

    ms_mixed, _ = timed(mixed, args.steps, args.warmup, torch)
    state_bytes = n_req * lay.h_v * lay.d_v * lay.d_k * 4
    return dict(n_req=n_req, w_tok=w_tok, ms_verify=ms_verify, ms_rec_verify=ms_rec_verify, ms_restore=ms_restore,
                state_bytes=state_bytes, lengths=lengths, ms_mixed=ms_mixed, t_live=int(sum(lengths)))


def device_prefill_inputs(torch, I, lay, lengths, seed, *, state_std=None, tail_std=None):
    """Seeded draws made on the device with the recipe of harness/inputs.py
    (x, z ~ N(0,1) and conv w ~ N(0, 0.5) as bf16; beta = sigmoid(N(0,1));
    g = -exp(A) softplus(N(0,1)) with A ~ U(0, ln 16) per v-head; norm w =
    1 + 0.1 N(0,1); states N(0, state_std), tails N(0, tail_std) or zero), for
    shapes whose host draws would take minutes.  Not the host stream's values:
    timing only."""
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    T, n, ch = int(sum(lengths)), len(lengths), lay.channels

    def rn(*shape, std=1.0):
        return torch.randn(*shape, generator=gen, device=dev) * std

    a_head = torch.rand(lay.h_v, generator=gen, device=dev) * math.log(16.0)
    d = dict(x=rn(T, ch).to(torch.bfloat16), w=rn(ch, 4, std=0.5).to(torch.bfloat16),
             beta=torch.sigmoid(rn(T, lay.h_v)),
             g=-torch.exp(a_head)[None, :] * torch.nn.functional.softplus(rn(T, lay.h_v)),
             z=rn(T, lay.h_v, lay.d_v).to(torch.bfloat16), nw=1.0 + 0.1 * rn(lay.d_v),
             cu=torch.from_numpy(I.cu_from_lengths(lengths)).to(dev))
    d["tail"] = (rn(n, 3, ch, std=tail_std) if tail_std is not None else torch.zeros(n, 3, ch, device=dev)
                 ).to(torch.bfloat16)
    d["state"] = (rn(n, lay.h_v, lay.d_v, lay.d_k, std=state_std) if state_std is not None
                  else torch.zeros(n, lay.h_v, lay.d_v, lay.d_k, device=dev))
    return d


def varlen_leg(args, torch, ops, I):
    """Varlen packed prefill: 8 sequences of log-uniform lengths in [512,
    32768] (seed 3), nonzero initial states and conv tails carried in place;
    conv, chunked rule with final states and the fused norm, bf16 outputs."""
    lay = I.MODEL_LAYOUT
    dev = "cuda:0"
    lengths = I.c3_lengths()
    T = int(sum(lengths))
    d = device_prefill_inputs(torch, I, lay, lengths, 3, state_std=0.02, tail_std=1.0)
    y_conv = torch.empty((T, lay.channels), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, lay.h_v, lay.d_v), dtype=torch.bfloat16, device=dev)
    q, k, v = ops.qkv_views(y_conv, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    ws = torch.empty(ops.gdn_chunk_fwd_workspace_size(lay.h_qk, lay.h_v, lay.d_k, lay.d_v, lay.chunk, len(lengths),
                                                      T, torch.bfloat16, True), dtype=torch.uint8, device=dev)

    def step(i):
        ops.gdn_conv1d_fwd(d["x"], d["w"], d["tail"], y_conv, cu_seqlens=d["cu"])
        ops.gdn_chunk_fwd(q, k, v, d["g"], d["beta"], y, chunk=lay.chunk, cu_seqlens=d["cu"],
                          initial_state=d["state"], final_state=d["state"], z=d["z"], norm_w=d["nw"], workspace=ws)

    def chunk_only(i):
        ops.gdn_chunk_fwd(q, k, v, d["g"], d["beta"], y, chunk=lay.chunk, cu_seqlens=d["cu"],
                          initial_state=d["state"], final_state=d["state"], workspace=ws)

    steps = max(2, args.steps // 4)
    ms, _ = timed(step, steps, 2, torch)
    ms_chunk, _ = timed(chunk_only, steps, 2, torch)
    return dict(lengths=lengths, T=T, ms=ms, ms_chunk=ms_chunk)


def long_context_leg(args, torch, ops, I):
    """Long-context chunked prefill then decode, one sequence: 16 calls of
    8192 tokens carrying the fp32 state and the conv history (fused norm, bf16
    outputs), then 256 batch-1 decode steps (conv step, recurrent step with
    the fused norm).  One run of the whole stream is one step."""
    lay = I.MODEL_LAYOUT
    dev = "cuda:0"
    n_calls, call_len, n_dec = 16, 8192, 256
    calls = [device_prefill_inputs(torch, I, lay, [call_len], 40 + i) for i in range(n_calls)]
    dec = device_prefill_inputs(torch, I, lay, [n_dec], 60)
    w, nw = calls[0]["w"], calls[0]["nw"]
    tail = torch.zeros((1, 3, lay.channels), dtype=torch.bfloat16, device=dev)
    state = torch.zeros((1, lay.h_v, lay.d_v, lay.d_k), device=dev)
    y_conv = torch.empty((call_len, lay.channels), dtype=torch.bfloat16, device=dev)
    y = torch.empty((call_len, lay.h_v, lay.d_v), dtype=torch.bfloat16, device=dev)
    q, k, v = ops.qkv_views(y_conv, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    yc1 = torch.empty((1, lay.channels), dtype=torch.bfloat16, device=dev)
    y1 = torch.empty((1, lay.h_v, lay.d_v), dtype=torch.bfloat16, device=dev)
    q1, k1, v1 = ops.qkv_views(yc1, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    ws = torch.empty(ops.gdn_chunk_fwd_workspace_size(lay.h_qk, lay.h_v, lay.d_k, lay.d_v, lay.chunk, 1, call_len,
                                                      torch.bfloat16, True), dtype=torch.uint8, device=dev)
    cu = calls[0]["cu"]
    stream = torch.cuda.current_stream()

    def prefill():
        for c in calls:
            ops.gdn_conv1d_fwd(c["x"], w, tail, y_conv, cu_seqlens=cu)
            ops.gdn_chunk_fwd(q, k, v, c["g"], c["beta"], y, chunk=lay.chunk, cu_seqlens=cu, initial_state=state,
                              final_state=state, z=c["z"], norm_w=nw, workspace=ws)

    def decode():
        for t in range(n_dec):
            ops.gdn_conv1d_fwd(dec["x"][t:t + 1], w, tail, yc1)
            ops.gdn_recurrent_step(q1, k1, v1, dec["g"][t:t + 1], dec["beta"][t:t + 1], state, y1,
                                   z=dec["z"][t:t + 1], norm_w=nw)

    def chunk_call(i):
        c = calls[i % n_calls]
        ops.gdn_chunk_fwd(q, k, v, c["g"], c["beta"], y, chunk=lay.chunk, cu_seqlens=cu, initial_state=state,
                          final_state=state, workspace=ws)

    def rec_step(i):
        t = i % n_dec
        ops.gdn_recurrent_step(q1, k1, v1, dec["g"][t:t + 1], dec["beta"][t:t + 1], state, y1)

    reps = 2
    prefill()
    decode()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    pre, dcd = [], []
    for _ in range(reps):
        state.zero_()
        tail.zero_()
        ev[0].record(stream)
        prefill()
        ev[1].record(stream)
        decode()
        ev[2].record(stream)
        torch.cuda.synchronize()
        pre.append(ev[0].elapsed_time(ev[1]))
        dcd.append(ev[1].elapsed_time(ev[2]))
    ms_chunk, _ = timed(chunk_call, 16, 2, torch)
    ms_rec, _ = timed(rec_step, 64, 4, torch)
    return dict(n_calls=n_calls, call_len=call_len, n_dec=n_dec, ms_prefill=min(pre), ms_decode=min(dcd),
                ms_chunk=ms_chunk, ms_rec=ms_rec)


def cpu_baseline(np, I, R):
    """The float64 oracle timed on this host's cores on bounded samples of the
    four workloads, all 32 v-heads, fewer tokens (the oracle walks tokens in
    order at a cost per token that does not depend on sequence length, so a
    rate in tokens/s carries over; decode steps scale with the request
    count), once with one thread and once with every core the process may use:
      prefill 4096     the whole single-sequence prefill mixer (conv, recurrence, norm)
      decode 64        16 of the 64 decode requests x 16 steps (steps/s scaled to 64 requests)
      varlen 8         the 8 packed sequences cut to 256 tokens each, nonzero states and tails
      long context     4096 tokens of the stream, and 32 batch-1 decode steps
    Rates are for the whole workload: tokens/s, or steps/s for decode."""
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    lay = I.MODEL_LAYOUT
    affinity = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else list(range(os.cpu_count()))
    kw = dict(h_qk=lay.h_qk, h_v=lay.h_v, d_k=lay.d_k, d_v=lay.d_v, bf16_boundary=True)

    def prefill_rate(lengths, seed, state_std=None, tail_std=None):
        d = I.prefill_inputs(seed, lay, lengths, state_std=state_std, tail_std=tail_std)
        t0 = time.perf_counter()
        R.mixer_prefill(d["x"], d["conv_w"], d["tail"], d["state"], d["beta"], d["g"], d["z"], d["norm_w"],
                        d["cu_seqlens"], **kw)
        dt = time.perf_counter() - t0
        return sum(lengths) / dt, dt

    def decode_rate(n_req, n_steps, seed, full_req):
        d = I.decode_inputs(seed, lay, n_req, n_steps)
        tail, state = d["tail"].astype(np.float64), d["state"].copy()
        t0 = time.perf_counter()
        for t in range(n_steps):
            R.mixer_decode_step(d["x"][t], d["conv_w"], tail, state, d["beta"][t], d["g"][t], d["z"][t],
                                d["norm_w"], np.arange(n_req), **kw)
        dt = time.perf_counter() - t0
        return 1.0 / (dt / n_steps * full_req / n_req), dt

    def run_all():
        r, used = {}, 0.0
        for key, fn in (("prefill_4096_tokens_per_s", lambda: prefill_rate([4096], 1)),
                        ("decode_64_requests_steps_per_s", lambda: decode_rate(16, 16, 2, 64)),
                        ("varlen_8_sequences_tokens_per_s", lambda: prefill_rate([256] * 8, 3, state_std=0.02, tail_std=1.0)),
                        ("long_context_prefill_tokens_per_s", lambda: prefill_rate([4096], 4)),
                        ("long_context_decode_steps_per_s", lambda: decode_rate(1, 32, 5, 1))):
            r[key], t = fn()
            used += t
        return {k: round(v, 2) for k, v in r.items()}, used

    limit = (lambda n: threadpool_limits(limits=n)) if threadpool_limits else (lambda n: contextlib.nullcontext())
    with limit(1):
        one, t_one = run_all()
    with limit(len(affinity)):
        allc, t_all = run_all()
    return dict(value=allc["prefill_4096_tokens_per_s"], unit="tokens/s", cores=len(affinity), kind="oracle",
                sample="the whole B=1 T=4096 prefill mixer (conv, recurrence, norm), all 32 v-heads, float64, "
                       "all cores the process may use (BLAS threads)",
                cpu_count=os.cpu_count(), affinity=len(affinity), one_thread=one, all_cores=allc,
                cpu_seconds_sampled={"one_thread": round(t_one, 1), "all_cores": round(t_all, 1)})


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(the mixer runs on one GPU with no sharding).", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    from gated_deltanet_mixer_causal_amd import ops
    from harness import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ops.L.load()
    probes = None
    if args.copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        probes = streaming_probes(torch)
    pf = prefill_leg(args, torch, np, ops, I)
    T = pf["T"]
    lay = pf["layout"]
    tok_s = T / (pf["ms"] * 1e-3)
    flop = FLOP_PER_TOKEN_HEAD * lay.h_v * T
    chunk_tflops = flop / (pf["ms_chunk"] * 1e-3) / 1e12
    traffic = measured_traffic("gdn_chunk_fwd")
    out = {
        "metric": "GDN prefill tokens/s (% MFMA peak) + decode state GB/s (% HBM peak)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GDN mixer prefill: conv1d+SiLU -> chunked gated delta rule -> gated RMSNorm; "
                               "B=1 T=4096, 16 q/k heads, 32 v heads, d=128, chunk 64, bf16 in/out, fp32 state",
                   "global_batch": 1, "seq_len": T, "parallelism": "none (1 GPU)",
                   "buffer_sets_rotated": args.sets},
        "roofline": {"kernel": "gdn_chunk_fwd (k_chunk_prep + k_chunk_scan)", "bound": "mfma",
                     "achieved": round(chunk_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(chunk_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "avg_launch_ms": round(pf["ms_chunk"], 4),
                     "algorithmic_flop_per_launch": flop,
                     "per_call": pf["chunk_stats"]},
        "env": environment(torch),
    }
    mf = measured_mfma("gdn_chunk_fwd")
    if mf is not None:
        out["roofline"]["mfma_executed"] = {
            "bf16_flop_per_launch": mf[0], "f32_flop_per_launch": mf[1],
            "bf16_frac_of_peak": round(mf[0] / (pf["ms_chunk"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "source": "rocprofv3 SQ_INSTS_VALU_MFMA_MOPS_BF16 / _F32 x 512 FLOP (profiles/)"}
    if not args.no_decode:
        dc = decode_leg(args, torch, np, ops, I)
        gbs = 2 * dc["state_bytes"] / (dc["ms_rec"] * 1e-3) / 1e9
        alg = 2 * dc["state_bytes"] + dc["small"]
        out["decode"] = {
            "workload": "64 requests x 1 token, same head layout, fp32 state 32x128x128 per request",
            "state_GB_per_s": round(gbs, 1),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "mixer_steps_per_s": round(1e3 / dc["ms"], 1),
            "mall_warm_state_GB_per_s": round(2 * dc["state_bytes"] / (dc["ms_rec_warm"] * 1e-3) / 1e9, 1),
            "ms_per_mixer_step": round(dc["ms"], 4),
            "ms_per_mixer_step_one_launch": round(dc["ms_fused"], 4),
            "one_launch_vs_two_launch": round(dc["ms_fused"] / dc["ms"], 4),
            "roofline": {"kernel": "gdn_recurrent_step", "bound": "hbm",
                         "achieved": round(alg / (dc["ms_rec"] * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(alg / (dc["ms_rec"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("gdn_recurrent_step"), "avg_launch_ms": round(dc["ms_rec"], 4),
                         "algorithmic_bytes_per_launch": alg, "per_call": dc["rec_stats"]},
        }
    out["fused_gates"] = {
        "what": "gdn_chunk_fwd_gated / gdn_recurrent_step_gated: g = -exp(a_log) softplus(a), beta = sigmoid(b) "
                "formed in the kernels from bf16 raw a|b projections (no g/beta tensors)",
        "chunk_fwd_ms": round(pf["ms_chunk_gated"], 4),
        "chunk_fwd_vs_plain": round(pf["ms_chunk_gated"] / pf["ms_chunk"], 4),
    }
    if not args.no_decode:
        out["fused_gates"]["recurrent_step_ms"] = round(dc["ms_rec_gated"], 4)
        out["fused_gates"]["recurrent_step_vs_plain"] = round(dc["ms_rec_gated"] / dc["ms_rec"], 4)
    if pf["ms_bwd"] is not None:
        out["backward"] = {
            "what": "gdn_chunk_bwd: dq, dk, dv, dg, dbeta, d_initial of the same 4096-token call (fp32 outputs; the chunked matrix-core form for these bf16 inputs)",
            "ms_per_call": round(pf["ms_bwd"], 4),
            "tokens_per_s": round(T / (pf["ms_bwd"] * 1e-3), 1),
            "vs_forward_chunk_fwd": round(pf["ms_bwd"] / pf["ms_chunk"], 2),
            "gdn_conv1d_bwd_ms": round(pf["ms_conv_bwd"], 4),
            "gdn_conv1d_bwd_GB_per_s": round(T * lay.channels * (2 + 4 + 4) / (pf["ms_conv_bwd"] * 1e-3) / 1e9, 1),
        }
    if not args.no_serving:
        sv = serving_leg(args, torch, np, ops, I)
        # recurrent verify: the live state read once, W checkpoint columns written
        vbytes = sv["state_bytes"] * (1 + sv["w_tok"])
        vgbs = vbytes / (sv["ms_rec_verify"] * 1e-3) / 1e9
        out["serving"] = {
            "verify": {"workload": f"{sv['n_req']} requests x {sv['w_tok']} draft tokens, eight checkpoint columns, "
                                   "fused norm, bf16 outputs",
                       "ms_per_round": round(sv["ms_verify"], 4),
                       "gdn_recurrent_verify_ms": round(sv["ms_rec_verify"], 4),
                       "gdn_recurrent_verify_state_GB_per_s": round(vgbs, 1),
                       "frac_hbm_peak": round(vgbs / PEAK_HBM_GBS, 4),
                       "restore_ms": round(sv["ms_restore"], 4),
                       "restore_GB_per_s": round(2 * sv["state_bytes"] / (sv["ms_restore"] * 1e-3) / 1e9, 1)},
            "mixed": {"workload": "one batch: 4 prompt chunks x 1024 tokens (2 fresh) + 60 decode tokens, "
                                  "slot-mapped pools of 128 rows, conv + chunked rule + fused norm, bf16 outputs",
                      "ms_per_batch": round(sv["ms_mixed"], 4),
                      "tokens_per_s": round(sv["t_live"] / (sv["ms_mixed"] * 1e-3), 1)},
            "buffer_sets": 1,
        }
    if not args.no_workloads:
        vl = varlen_leg(args, torch, ops, I)
        vflop = FLOP_PER_TOKEN_HEAD * lay.h_v * vl["T"]
        vtf = vflop / (vl["ms_chunk"] * 1e-3) / 1e12
        out["varlen"] = {
            "workload": f"8 packed sequences {vl['lengths']} ({vl['T']} tokens), nonzero states and conv tails, "
                        "conv + chunked rule + fused norm, bf16 outputs, final states in place",
            "tokens_per_s": round(vl["T"] / (vl["ms"] * 1e-3), 1), "ms_per_step": round(vl["ms"], 4),
            "roofline": {"kernel": "gdn_chunk_fwd", "bound": "mfma", "achieved": round(vtf, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(vtf / PEAK_BF16_TFLOPS, 4),
                         "avg_launch_ms": round(vl["ms_chunk"], 4), "algorithmic_flop_per_launch": vflop}}
        lc = long_context_leg(args, torch, ops, I)
        cflop = FLOP_PER_TOKEN_HEAD * lay.h_v * lc["call_len"]
        ctf = cflop / (lc["ms_chunk"] * 1e-3) / 1e12
        sb1 = lay.h_v * lay.d_v * lay.d_k * 4
        rec_alg = 2 * sb1 + (2 * lay.h_qk * lay.d_k * 2 + lay.h_v * lay.d_v * 2 + 2 * lay.h_v * 4)
        out["long_context"] = {
            "workload": f"one sequence: {lc['n_calls']} chunked-prefill calls of {lc['call_len']} tokens carrying the "
                        f"fp32 state and conv history (fused norm, bf16), then {lc['n_dec']} batch-1 decode steps",
            "prefill_tokens_per_s": round(lc["n_calls"] * lc["call_len"] / (lc["ms_prefill"] * 1e-3), 1),
            "prefill_ms": round(lc["ms_prefill"], 3),
            "decode_steps_per_s": round(lc["n_dec"] / (lc["ms_decode"] * 1e-3), 1),
            "decode_ms": round(lc["ms_decode"], 3),
            "roofline": {"kernel": "gdn_chunk_fwd (one 8192-token call)", "bound": "mfma", "achieved": round(ctf, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ctf / PEAK_BF16_TFLOPS, 4),
                         "avg_launch_ms": round(lc["ms_chunk"], 4), "algorithmic_flop_per_launch": cflop},
            "decode_roofline": {"kernel": "gdn_recurrent_step (1 request)", "bound": "hbm",
                                "achieved": round(rec_alg / (lc["ms_rec"] * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(rec_alg / (lc["ms_rec"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
                                "avg_launch_ms": round(lc["ms_rec"], 4), "algorithmic_bytes_per_launch": rec_alg,
                                "note": "2 MiB of state per step: launch-latency bound, far from the HBM roof"}}
    if probes is not None:
        out["streaming_probes"] = probes
    if not args.no_cpu_baseline:
        from oracle import gdn_ref as R
        out["cpu_baseline"] = cpu_baseline(np, I, R)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
