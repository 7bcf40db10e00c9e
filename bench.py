"""Benchmark of the gated delta rule hot path on one MI355X.

A step is one pass of the path over one batch of synthetic input:
  * prefill: kda_prefill_chunked on the long-context workload
    (B=1, H=16, d_k=d_v=128, T=262144, bf16 q/k/v, scalar alpha, C=64),
    emitting o and the final state -- `value` is its throughput in tokens/s;
  * decode: kda_decode_step on the batched-decode workload (B=256, H=16,
    d=128, per-key alpha, fp32 state updated in place) -- reported in
    `decode.us_per_step`.
Inputs are generated on the GPU (seeded) and resident in HBM before timing.
Kernel durations come from HIP events on the stream the kernels are launched
on (torch's current stream). Roofline figures use algorithmic bytes and flops:
  prefill bytes = q,k,v (bf16) + alpha + beta + o (fp32) + final state,
  prefill flops per chunk-head = 6 C dk dv + 3 C^2 dk + 2 C^2 dv + C^3/3,
  decode bytes = state read + write + q,k,v + alpha + beta + o.
The CPU baseline is the fp64 oracle on the host's cores over a bounded
token prefix of the same prefill workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s @T=256K H16 d128; decode µs/step @B256; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, TFLOP/s
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA, TFLOP/s


def prefill_algorithmic(T, H, dk, dv, n_seqs, per_key, qkv_bytes=2, C=64, with_init=False, n_snap=0):
    b = T * H * (2 * dk + dv) * qkv_bytes          # q, k, v
    b += T * H * (dk if per_key else 1) * 4        # alpha
    b += T * H * 4                                 # beta
    b += T * H * dv * 4                            # o
    b += n_seqs * H * dv * dk * 4                  # final state
    if with_init:
        b += n_seqs * H * dv * dk * 4
    b += n_snap * H * dv * dk * 4
    chunks = T / C                                 # full chunks (all configs are multiples of 64 here)
    f = chunks * H * (6 * C * dk * dv + 3 * C * C * dk + 2 * C * C * dv + C ** 3 / 3)
    return b, f


def backward_algorithmic(T, H, d, n_seqs, per_key, qkv_bytes=2, C=64, with_init=False, with_final=False):
    """Bytes: q, k, v, alpha, beta and d_o read once, dq, dk, dv, dalpha, dbeta
    (fp32) written once (plus the states when given/wanted). Flops per
    (chunk, head) of the chunked backward's products (dense, the lower
    triangles of Bm and dBm at half): 18 C d^2 + 26 C^2 d + (13/3) C^3; the
    forward recomputed for the chunk-start states is not counted."""
    a_el = d if per_key else 1
    b = T * H * 3 * d * qkv_bytes + T * H * (a_el + 1) * 4 + T * H * d * 4        # inputs, d_o
    b += T * H * 3 * d * 4 + T * H * (a_el + 1) * 4                               # gradients
    b += n_seqs * H * d * d * 4 * (1 + int(with_init) + int(with_final))          # d_init (+ init, d_final)
    f = (T / C) * H * (18 * C * d * d + 26 * C * C * d + 13 / 3 * C ** 3)
    return b, f


def decode_algorithmic(B, H, dk, dv, per_key, qkv_bytes=2):
    b = 2 * B * H * dv * dk * 4                    # state read + write
    b += B * H * (2 * dk + dv) * qkv_bytes
    b += B * H * (dk if per_key else 1) * 4 + B * H * 4 + B * H * dv * 4
    f = B * H * dv * (7 * dk)                      # decay, 2 dots, update, read-out
    return b, f


def kernel_sources_digest() -> str:
    """sha256 over the kernel sources and headers: HBM counter figures stored
    under profiles/ are only reported while the kernels they were taken on are
    unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_72_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".h")):
            h.update(fn.encode())
            h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(name: str):
    """HBM bytes per launch from the counter summary profiles/<name>_traffic.md
    (FETCH_SIZE and WRITE_SIZE passes, each scaled by the plain-copy
    calibration), or None if it is missing or was taken on other kernel sources."""
    import re
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^sources_sha256_16:\s*([0-9a-f]{16})\s*$", text, flags=re.M)
    b = re.search(r"^traffic_bytes_per_launch:\s*([0-9]+)\s*$", text, flags=re.M)
    if not m or not b or m.group(1) != kernel_sources_digest():
        return None
    return int(b.group(1))


def stored_mfma(name: str):
    """MFMA busy percentage per kernel of a workload's prefill, from the
    counter summary profiles/mfma_activity_prefill.md (rocprofv3 pass over
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE), or None if it is missing or
    was taken on other kernel sources."""
    import re
    path = os.path.join(ROOT, "profiles", "mfma_activity_prefill.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^sources_sha256_16:\s*([0-9a-f]{16})\s*$", text, flags=re.M)
    if not m or m.group(1) != kernel_sources_digest():
        return None
    out = {}
    for k, v in re.findall(r"^mfma_busy_pct " + re.escape(name) + r" (\S+): ([0-9.]+)$", text, flags=re.M):
        out[k] = float(v)
    return out or None


def measure_ceilings(torch, reps: int = 5) -> dict:
    """Measured device ceilings (libkda_calib.so, include/kda_calib.h): a
    streaming 16-byte copy of 1 GiB and a dense fp16 MFMA loop, each timed with
    HIP events; the best of `reps` runs."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_delta_rule_72_amd", "libkda_calib.so"))
    lib.kda_calib_mfma_f16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.kda_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_void_p]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    n_vec = 1 << 26                                   # 1 GiB in 16-byte vectors
    src = torch.ones(n_vec * 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    blocks_mfma, iters = 1024, 20000
    out = torch.empty(blocks_mfma * 256 * 4, dtype=torch.float32, device=dev)

    def timed(fn):
        best = float("inf")
        for _ in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = fn()
            b.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"calibration kernel failed with status {rc}")
            best = min(best, a.elapsed_time(b))
        return best

    copy_ms = timed(lambda: lib.kda_calib_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                               n_vec, 256 * 32, sp))
    mfma_ms = timed(lambda: lib.kda_calib_mfma_f16(blocks_mfma, iters, ctypes.c_void_p(out.data_ptr()), sp))
    flops = blocks_mfma * 4 * iters * 8 * 16384
    del src, dst, out
    return {"copy_GBs": round(2 * n_vec * 16 / (copy_ms * 1e-3) / 1e9, 1),
            "mfma_f16_TFLOPs": round(flops / (mfma_ms * 1e-3) / 1e12, 1),
            "how": "best of 5: 1 GiB streaming copy, 8192 workgroups x 256 threads x 4 nontemporal "
                   "16-byte vectors per step (read + write counted); "
                   "fp16 16x16x32 MFMA loop, 1024 workgroups x 4 wavefronts x 8 independent chains"}


def time_prefill(kda, torch, inp, w, steps, warmup, snaps_on_host=False):
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    dev = inp["q"].device
    shape = kda.make_shape(H, dk, dv, inp["q"].dtype, w.gate == "per_key")
    cu_h = inp["cu_seqlens_host"]
    o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    fin = torch.empty((w.num_seqs, H, dv, dk), dtype=torch.float32, device=dev)
    n_snap = kda.kda_snapshot_count(cu_h, w.interval)
    snaps = None
    if n_snap:
        snaps = (torch.empty((n_snap, H, dv, dk), dtype=torch.float32, pin_memory=True) if snaps_on_host
                 else torch.empty((n_snap, H, dv, dk), dtype=torch.float32, device=dev))
    ws = torch.empty(max(kda.kda_prefill_workspace_size(shape, cu_h, 64, w.interval), 1),
                     dtype=torch.uint8, device=dev)

    def call():
        kda.kda_prefill_chunked(shape, cu_h, inp["cu_seqlens"], inp["q"], inp["k"], inp["v"],
                                inp["alpha"], inp["beta"], inp["initial_state"], o, fin, snaps, ws,
                                snapshot_interval=w.interval)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        call()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [s.elapsed_time(e) for s, e in ev]
    return ms, wall


def time_decode(kda, torch, w, steps, warmup, n_buffers=4):
    from gated_delta_rule_72_amd import workloads as wl
    dev = torch.device("cuda:0")
    bufs = [wl.make_decode_inputs(w, dev, seed=w.seed + i) for i in range(n_buffers)]
    outs = [torch.empty((w.num_seqs, w.H, w.dv), dtype=torch.float32, device=dev) for _ in bufs]
    shape = kda.make_shape(w.H, w.dk, w.dv, bufs[0]["q"].dtype, w.gate == "per_key")

    def call(i):
        d = bufs[i % n_buffers]
        kda.kda_decode_step(shape, w.num_seqs, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state"],
                            outs[i % n_buffers])

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (s, e) in enumerate(ev):
        s.record(stream)
        call(i)
        e.record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def time_decode_tokens(kda, torch, w, n_tok, steps, warmup, keep_states, n_buffers=4):
    """kda_decode_tokens over n_tok tokens per sequence of the decode workload,
    committing every token; optionally writing the per-token states."""
    from gated_delta_rule_72_amd import workloads as wl
    dev = torch.device("cuda:0")
    B = w.num_seqs
    ws = w.with_(seq_lens=(n_tok,) * B)
    bufs = []
    for i in range(n_buffers):
        inp = wl.make_prefill_inputs(ws, dev, seed=w.seed + 100 + i)
        x = {y: inp[y].view(B, n_tok, *inp[y].shape[1:]) for y in ("q", "k", "v", "alpha", "beta")}
        x["state"] = inp["initial_state"]
        bufs.append(x)
    shape = kda.make_shape(w.H, w.dk, w.dv, bufs[0]["q"].dtype, w.gate == "per_key")
    o = torch.empty((B, n_tok, w.H, w.dv), dtype=torch.float32, device=dev)
    ts = torch.empty((B, n_tok, w.H, w.dv, w.dk), dtype=torch.float32, device=dev) if keep_states else None

    def call(i):
        d = bufs[i % n_buffers]
        kda.kda_decode_tokens(shape, B, n_tok, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state"], o, ts)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (s0, e0) in enumerate(ev):
        s0.record(stream)
        call(i)
        e0.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    del bufs, o, ts
    torch.cuda.empty_cache()
    return ms


def layer_algorithmic(T, H, d, n_seqs, per_key, qkv_bytes=2, out_bytes=2):
    """Bytes the layer front and back end must move once each: front reads
    xq, xk, xv, the gate logits, the taps and the carried conv state and writes
    q, k, v, alpha, beta and the new conv state; back reads o and the gate
    logits (fp32) and writes the output."""
    rows = T * H
    a_el = rows * (d if per_key else 1)
    front = (2 * 3 * rows * d * qkv_bytes + 2 * a_el * 4 + 2 * rows * 4 + 3 * H * d * 4 * 4
             + 2 * n_seqs * 9 * H * d * qkv_bytes + (n_seqs + 1) * 8)
    back = rows * d * (4 + 4 + out_bytes) + d * 4
    return front, back


def time_layer(kda, torch, w, steps, warmup):
    """HIP-event times of kda_layer_front (with carried conv state in and out)
    and kda_layer_back, of front + kda_prefill_chunked + back, and of front +
    kda_layer_prefill (the recurrence and the back end in one call, gate
    logits in the q/k/v dtype)."""
    from gated_delta_rule_72_amd import workloads as wl
    dev = torch.device("cuda:0")
    li = wl.make_layer_inputs(w, dev)
    pinp = wl.make_prefill_inputs(w, dev)
    T, H, d = w.T, w.H, w.dk
    shape = kda.make_shape(H, d, d, li["xq"].dtype, w.gate == "per_key")
    q, k, v = (torch.empty_like(li["xq"]) for _ in range(3))
    alpha = torch.empty_like(li["alpha_logit"])
    beta = torch.empty_like(li["beta_logit"])
    st = torch.empty_like(li["conv_state"])
    out = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    cu_h = li["cu_seqlens_host"]
    o = torch.empty((T, H, d), dtype=torch.float32, device=dev)
    fin = torch.empty((w.num_seqs, H, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(kda.kda_prefill_workspace_size(shape, cu_h, 64, 0), 1), dtype=torch.uint8, device=dev)
    g_qkv = li["g_logit"].to(li["xq"].dtype)
    ws_l = torch.empty(max(kda.kda_layer_prefill_workspace_size(shape, cu_h, 64, 0), 1), dtype=torch.uint8,
                       device=dev)

    def front():
        kda.kda_layer_front(shape, cu_h, li["cu_seqlens"], li["xq"], li["xk"], li["xv"], li["conv_w"],
                            li["conv_state"], li["alpha_logit"], 5.0, li["beta_logit"], q, k, v, alpha, beta, st)

    def back(src):
        kda.kda_layer_back(shape, T, src, li["g_logit"], li["norm_w"], 1e-6, kda.KDA_BF16, out)

    def layer():
        front()
        kda.kda_prefill_chunked(shape, cu_h, li["cu_seqlens"], q, k, v, alpha, beta, pinp["initial_state"],
                                o, fin, None, ws)
        back(o)

    def layer_one_call():
        front()
        kda.kda_layer_prefill(shape, cu_h, li["cu_seqlens"], q, k, v, alpha, beta, pinp["initial_state"], g_qkv,
                              li["norm_w"], 1e-6, kda.KDA_BF16, out, fin, None, ws_l)

    res = {}
    stream = torch.cuda.current_stream()
    for name, fn in (("front", front), ("back", lambda: back(li["o"])), ("layer", layer),
                     ("layer_one_call", layer_one_call)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for s_, e_ in ev:
            s_.record(stream)
            fn()
            e_.record(stream)
        torch.cuda.synchronize()
        ms = [s_.elapsed_time(e_) for s_, e_ in ev]
        res[name] = sum(ms) / len(ms)
    del li, pinp
    torch.cuda.empty_cache()
    return res


def time_backward(kda, torch, w, steps, warmup):
    """HIP-event time of kda_prefill_backward (outputs and workspace allocated
    beforehand; the recomputed forward is inside the call)."""
    from gated_delta_rule_72_amd import workloads as wl
    dev = torch.device("cuda:0")
    inp = wl.make_prefill_inputs(w, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 11)
    d_o = torch.randn((w.T, w.H, w.dv), generator=g, device=dev)
    shape = kda.make_shape(w.H, w.dk, w.dv, inp["q"].dtype, w.gate == "per_key")
    cu_h = inp["cu_seqlens_host"]
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty((w.T, w.H, w.dk), **f32) for _ in range(3))
    da = torch.empty(inp["alpha"].shape, **f32)
    db = torch.empty((w.T, w.H), **f32)
    di = torch.empty((w.num_seqs, w.H, w.dv, w.dk), **f32)
    ws_bytes = kda.kda_prefill_backward_workspace_size(shape, cu_h)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def call():
        kda.kda_prefill_backward(shape, cu_h, inp["cu_seqlens"], inp["q"], inp["k"], inp["v"], inp["alpha"],
                                 inp["beta"], inp["initial_state"], d_o, None, dq, dk, dv, da, db, di, ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s_, e_ in ev:
        s_.record(stream)
        call()
        e_.record(stream)
    torch.cuda.synchronize()
    ms = [s_.elapsed_time(e_) for s_, e_ in ev]
    with_init = inp["initial_state"] is not None
    del inp, d_o, dq, dk, dv, da, db, di, ws
    torch.cuda.empty_cache()
    return sum(ms) / len(ms), ws_bytes, with_init


def cpu_baseline(w, inp, tokens: int):
    """fp64 oracle on the host over the first `tokens` tokens of the workload."""
    tokens = min(tokens, w.T)
    from gated_delta_rule_72_amd import workloads as wl
    import oracle
    sl = slice(0, tokens)
    A = {n: wl.to_oracle_arrays(inp[n][sl]) for n in ("q", "k", "v", "alpha", "beta")}
    import numpy as np
    t0 = time.perf_counter()
    rc, rep = oracle.ref_check(A["q"], A["k"], A["v"], A["alpha"], A["beta"],
                               np.array([0, tokens], np.int64), None, 0)
    secs = time.perf_counter() - t0
    return {"value": tokens / secs, "unit": "tokens/s", "cores": int(rep["threads"]), "kind": "oracle",
            "sample": (f"first {tokens} of {w.T} tokens" if tokens < w.T else f"all {w.T} tokens")
                      + f" of {w.name}, all {w.H} heads, fp64 token-by-token recurrence",
            "seconds": round(secs, 3), "cpu_model": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (first "model name" of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-tokens", type=int, default=262144,
                    help="token prefix the CPU oracle baseline runs on (0 = skip)")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="profiling: only the prefill loop")
    ap.add_argument("--prefill-workload", default="long_prefill_T262144_H16_d128",
                    help="workload name for the prefill line (default: the headline long prefill)")
    ap.add_argument("--decode-only", action="store_true", help="profiling: only the decode loop")
    ap.add_argument("--no-other-prefill", action="store_true",
                    help="skip timing the other prefill workloads (KDA layer shape, varlen pack)")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward pass")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip timing the KDA layer front and back end")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="profiling: copy a 256 MiB fp32 buffer 3 times (known bytes for HBM counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the path runs on a "
              f"single GPU (sequences and heads would shard across GPUs without exchange).", file=sys.stderr)
        return 2

    import torch
    import gated_delta_rule_72_amd as kda
    from gated_delta_rule_72_amd import workloads as wl

    kda.load()
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_copy": src.numel() * 4,
                          "bytes_written_per_copy": dst.numel() * 4, "copies": 3}))
        return 0
    if args.decode_only:
        d = wl.DECODE
        dms = time_decode(kda, torch, d, max(args.steps, 20), args.warmup)
        davg = sum(dms) / len(dms)
        print(json.dumps({"decode_us_per_step": davg * 1e3, "steps": len(dms)}))
        return 0
    ceilings = measure_ceilings(torch)
    w = wl.ALL[args.prefill_workload]
    inp = wl.make_prefill_inputs(w, dev)
    torch.cuda.synchronize()
    ms, wall = time_prefill(kda, torch, inp, w, args.steps, args.warmup)
    ms_avg = sum(ms) / len(ms)
    n_snap = kda.kda_snapshot_count(inp["cu_seqlens_host"], w.interval)
    pb, pf = prefill_algorithmic(w.T, w.H, w.dk, w.dv, w.num_seqs, w.gate == "per_key",
                                 qkv_bytes=2 if w.dtype == "bf16" else 4,
                                 with_init=inp["initial_state"] is not None, n_snap=n_snap)
    gbs = pb / (ms_avg * 1e-3) / 1e9
    tfl = pf / (ms_avg * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": w.T / (ms_avg * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_avg,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16-mfma/fp32-state",
        "data": "synthetic (seeded; no dataset)",
        "config": {"workload": w.name, "B": w.num_seqs, "T": w.T, "H": w.H, "d_k": w.dk, "d_v": w.dv,
                   "gate": w.gate, "chunk": w.chunk, "qkv": w.dtype, "snapshot_interval": w.interval},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": stored_traffic(w.name),
                     "mfma_busy_pct_counters": stored_mfma(w.name),
                     "kernel": "kda_prefill_chunked = prefill_map_chain_kernel pass 1 + segment_scan + "
                               "prefill_wu_pipe_kernel pass 3 (automatic segment plan; one sequence, so the "
                               "kernels form their work items and no work-table kernel runs)",
                     "algorithmic_bytes_per_launch": int(pb), "algorithmic_flops_per_launch": int(pf),
                     "frac_of_measured_copy": round(gbs / ceilings["copy_GBs"], 4),
                     "mfma_tflops": round(tfl, 2), "mfma_frac": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
                     "attainable_frac": round((pb / (HBM_PEAK_GBS * 1e9)) / (ms_avg * 1e-3), 4)},
        "prefill_ms": {"avg": ms_avg, "median": sorted(ms)[len(ms) // 2], "min": min(ms), "max": max(ms),
                       "timing": "HIP events on the launch stream around each kda_prefill_chunked call"},
        "kernel_level": "hip-gfx950-chunked-v1",
        "kernel_sources_sha256_16": kernel_sources_digest(),
        "measured_ceilings": ceilings,
    }
    del inp
    torch.cuda.empty_cache()
    if not args.no_other_prefill and not args.prefill_only:
        other = {}
        for ow in (wl.KDA_LAYER, wl.VARLEN):
            oinp = wl.make_prefill_inputs(ow, dev)
            torch.cuda.synchronize()
            oms, _ = time_prefill(kda, torch, oinp, ow, max(5, args.steps // 2), args.warmup)
            oavg = sum(oms) / len(oms)
            on_snap = kda.kda_snapshot_count(oinp["cu_seqlens_host"], ow.interval)
            ob, of = prefill_algorithmic(ow.T, ow.H, ow.dk, ow.dv, ow.num_seqs, ow.gate == "per_key",
                                         qkv_bytes=2 if ow.dtype == "bf16" else 4,
                                         with_init=oinp["initial_state"] is not None, n_snap=on_snap)
            ogbs = ob / (oavg * 1e-3) / 1e9
            other[ow.name] = {"ms_per_call": round(oavg, 4), "tokens_per_s": round(ow.T / (oavg * 1e-3), 1),
                              "hbm_GBs": round(ogbs, 1), "hbm_frac": round(ogbs / HBM_PEAK_GBS, 4),
                              "mfma_frac": round(of / (oavg * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                              "algorithmic_bytes": int(ob), "algorithmic_flops": int(of), "calls": len(oms),
                              "mfma_busy_pct_counters": stored_mfma(ow.name)}
            if on_snap:
                hms, _ = time_prefill(kda, torch, oinp, ow, max(5, args.steps // 2), args.warmup, snaps_on_host=True)
                other[ow.name]["ms_per_call_snapshots_to_pinned_host"] = round(sum(hms) / len(hms), 4)
                other[ow.name]["snapshot_bytes_to_host"] = on_snap * ow.H * ow.dv * ow.dk * 4
            del oinp
            torch.cuda.empty_cache()
        result["other_prefill"] = other
    if not args.no_layer and not args.prefill_only:
        layer = {}
        for lw in (wl.KDA_LAYER, wl.LONG_PREFILL):
            t = time_layer(kda, torch, lw, max(5, args.steps // 2), args.warmup)
            fb, bb = layer_algorithmic(lw.T, lw.H, lw.dk, lw.num_seqs, lw.gate == "per_key",
                                       qkv_bytes=2 if lw.dtype == "bf16" else 4)
            layer[lw.name] = {
                "front_us": round(t["front"] * 1e3, 2), "back_us": round(t["back"] * 1e3, 2),
                "front_hbm_GBs": round(fb / (t["front"] * 1e-3) / 1e9, 1),
                "back_hbm_GBs": round(bb / (t["back"] * 1e-3) / 1e9, 1),
                "front_hbm_frac": round(fb / (t["front"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "back_hbm_frac": round(bb / (t["back"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "front_algorithmic_bytes": int(fb), "back_algorithmic_bytes": int(bb),
                "front_recurrence_back_ms": round(t["layer"], 4),
                "front_recurrence_back_tokens_per_s": round(lw.T / (t["layer"] * 1e-3), 1),
                "front_then_layer_prefill_ms": round(t["layer_one_call"], 4),
                "front_then_layer_prefill_tokens_per_s": round(lw.T / (t["layer_one_call"] * 1e-3), 1),
                "layer_prefill_back_end_fused": bool(lw.dk == 128 and lw.dtype == "bf16" and lw.gate == "scalar")}
        result["layer_front_back"] = layer
    if not args.no_backward and not args.prefill_only:
        bwd = {}
        for bw in (wl.KDA_LAYER, wl.LONG_PREFILL, wl.VARLEN):
            bms, ws_bytes, with_init = time_backward(kda, torch, bw, max(3, args.steps // 5), 1)
            bb, bf = backward_algorithmic(bw.T, bw.H, bw.dk, bw.num_seqs, bw.gate == "per_key",
                                          qkv_bytes=2 if bw.dtype == "bf16" else 4, with_init=with_init)
            tfl = bf / (bms * 1e-3) / 1e12
            bwd[bw.name] = {"ms_per_call": round(bms, 4), "tokens_per_s": round(bw.T / (bms * 1e-3), 1),
                            "roofline": {"bound": "mfma", "achieved": round(tfl, 2), "peak": MFMA_F32_PEAK_TFLOPS,
                                         "unit": "TFLOP/s", "frac": round(tfl / MFMA_F32_PEAK_TFLOPS, 4),
                                         "dtype": "fp32 MFMA"},
                            "algorithmic_flops": int(bf), "algorithmic_bytes": int(bb),
                            "hbm_frac": round(bb / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "workspace_bytes": int(ws_bytes),
                            "includes": "forward recompute (states every 64 tokens) + backward kernels"}
        result["backward"] = bwd
    if not args.skip_decode and not args.prefill_only:
        d = wl.DECODE
        dms = time_decode(kda, torch, d, max(args.steps, 20), args.warmup)
        davg = sum(dms) / len(dms)
        db, df = decode_algorithmic(d.num_seqs, d.H, d.dk, d.dv, d.gate == "per_key")
        dgbs = db / (davg * 1e-3) / 1e9
        result["decode"] = {"workload": d.name, "us_per_step": davg * 1e3,
                            "us_median": sorted(dms)[len(dms) // 2] * 1e3, "us_min": min(dms) * 1e3,
                            "roofline": {"bound": "hbm", "achieved": round(dgbs, 1), "peak": HBM_PEAK_GBS,
                                         "unit": "GB/s", "frac": round(dgbs / HBM_PEAK_GBS, 4),
                                         "frac_of_measured_copy": round(dgbs / ceilings["copy_GBs"], 4),
                                         "traffic": stored_traffic(d.name),
                                         "algorithmic_bytes_per_launch": int(db)},
                            "kernel_level": "hip-gfx950-decode-v1"}
        n_draft = 4
        draft = {}
        for keep in (False, True):
            tms = time_decode_tokens(kda, torch, d, n_draft, max(args.steps, 20), args.warmup, keep)
            tavg = sum(tms) / len(tms)
            tb, _ = decode_algorithmic(d.num_seqs, d.H, d.dk, d.dv, d.gate == "per_key")
            st_bytes = 2 * d.num_seqs * d.H * d.dv * d.dk * 4
            tb = st_bytes + n_draft * (tb - st_bytes)          # state once, per-token inputs and o
            if keep:
                tb += n_draft * st_bytes // 2                   # one state written per token
            tgbs = tb / (tavg * 1e-3) / 1e9
            draft["with_token_states" if keep else "commit_only"] = {
                "us_per_call": round(tavg * 1e3, 2), "us_per_token": round(tavg * 1e3 / n_draft, 2),
                "hbm_GBs": round(tgbs, 1), "hbm_frac": round(tgbs / HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_launch": int(tb)}
        result["decode_tokens"] = {"workload": f"{d.name}_x{n_draft}_tokens", "tokens_per_sequence": n_draft,
                                   **draft}
    if args.cpu_tokens > 0 and not args.prefill_only:
        inp = wl.make_prefill_inputs(w, dev)
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_tokens)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
