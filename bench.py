#!/usr/bin/env python3
"""Throughput of the RWKV-7 decode / prefill hot path on one MI355X.

Headline (the JSON line's `value`): decode tokens/s of the 2.9B-shape model
(32 layers, C 2560, 40 heads x 64, F 10240, V 65536, fp16 weights, fp32
state) at B = 1: a 64-token uniform-id prompt is prefilled (63 tokens, the
last one is the first decode input), then every timed step is one decode
step (rwkv7_decode_step) plus greedy selection (rwkv7_greedy) whose ids feed
the next step on the device.  Inputs are resident in HBM before timing.

Also in the same line:
  roofline     the dominant kernel's achieved HBM GB/s (algorithmic bytes per
               launch / average launch time from HIP events) against 8 TB/s
  step         algorithmic bytes per decode step / step time
  kernels      per-class time breakdown of one decode step (HIP events)
  batched      B = 64 / 256 decode of the 2.9B shape and B = 256 of the 7.2B
               shape (prompts of 20-2000 tokens, penalties 1.0 / 1.0, decay
               0.996) with per-projection MFMA TFLOP/s
  prefill      tokens/s of rwkv7_prefill_seq at T = 128 / 512 / 2048
  cpu_baseline the fp64 NumPy oracle timed on a bounded sample on the host

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA

METRIC = "decode tokens/sec at B=1/64/256 (2.9B-shape fp16) + % of HBM/MFMA roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic bytes
def class_bytes(s, B: int, nnz: int, sparse: bool, fused_value: bool = False, int8: bool = False):
    """Compulsory HBM bytes per launch of each kernel class for B decode rows:
    every weight read once, activations / state read and written once.  With
    the value fused into the key projection (B <= 2) the active value rows
    count in that kernel, and the fold only moves the residual.  int8: the
    GEMV-streamed matrices at one byte per weight plus a 4-byte scale per row
    (the adapters' second stage, read by the WKV kernel, stays fp16)."""
    C, F, V, H = s.n_embd, s.ffn, s.vocab, s.n_head
    if int8:
        b = class_bytes(s, B, nnz, sparse, fused_value)
        Din = s.d_w + s.d_a + s.d_v + s.d_g
        n_in = 3 * C + Din
        b["proj_in"] -= n_in * C - n_in * 4
        b["proj_out"] -= C * C - C * 4
        b["cmix_key"] -= F * C - F * 4
        if fused_value:
            b["cmix_key"] -= nnz * C - nnz * 4
        b["head"] -= V * C - V * 4
        return b
    Din = s.d_w + s.d_a + s.d_v + s.d_g
    n_in = 3 * C + Din
    ns = max(1, min(32, -(-512 // (C // 64))))
    b = {}
    b["ln_mix"] = B * C * 4 * 4 + B * C * 4 * 3.5            # x, shift r/w, mixed outs (avg of 6 and 1)
    b["proj_in"] = n_in * C * 2 + B * 6 * C * 4 + B * n_in * 4
    b["wkv"] = B * H * 64 * 64 * 4 * 2 + C * Din * 2 + B * (3 * C + Din + 2 * C) * 4
    b["proj_out"] = C * C * 2 + B * C * 4 * 3
    b["cmix_key"] = F * C * 2 + B * C * 4 + B * F * 4
    if sparse:
        b["cmix_value"] = nnz * C * 2 + B * F * 4 + ns * B * C * 4
    else:
        b["cmix_value"] = F * C * 2 + B * F * 2 + B * C * 4 * 2
    if fused_value:
        b["cmix_key"] += nnz * C * 2
        b["cmix_value"] = B * C * 4 * 2
    b["head"] = V * C * 2 + B * C * 4 + B * V * 4
    b["other"] = B * C * 2 + B * C * 4
    return b


def class_flops(s, B: int):
    C, F, V = s.n_embd, s.ffn, s.vocab
    Din = s.d_w + s.d_a + s.d_v + s.d_g
    return {"proj_in": 2 * B * (3 * C + Din) * C, "proj_out": 2 * B * C * C,
            "cmix_key": 2 * B * F * C, "cmix_value": 2 * B * F * C, "head": 2 * B * V * C}


def step_bytes(s, B, nnz, sparse, int8=False):
    # the same total with or without the fused value (int8 applies with it)
    cb = class_bytes(s, B, nnz, sparse, fused_value=int8, int8=int8)
    L = s.n_layer
    per_layer = 2 * cb["ln_mix"] + cb["proj_in"] + cb["wkv"] + cb["proj_out"] + cb["cmix_key"] + cb["cmix_value"]
    greedy = B * s.vocab * 4 * 3   # logits read, occurrences read + written
    return L * per_layer + cb["ln_mix"] + cb["head"] + cb["other"] + greedy


# ---------------------------------------------------------------- PMC traffic record
# source file of each B=1 kernel class (the traffic record is tied to its text)
KERNEL_SRC = {"proj_in": "k_gemv.hip", "cmix_key": "k_gemv.hip", "proj_out": "k_gemv.hip",
              "head": "k_gemv.hip", "cmix_value": "k_misc.hip", "wkv": "k_wkv.hip"}


def _src_hash(cls):
    import hashlib
    h = hashlib.sha256()
    for f in (KERNEL_SRC[cls], "common.h"):
        with open(os.path.join(ROOT, "rwkv_linear_attention_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel, cls):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (profiles/pmc_traffic_*.txt, copy-calibrated), or None when
    there is no record or the kernel's source changed since it was taken."""
    import glob
    import re
    if cls not in KERNEL_SRC:
        return None
    want = _src_hash(cls)
    for fn in sorted(glob.glob(os.path.join(ROOT, "profiles", "pmc_traffic_*.txt"))):
        with open(fn) as fh:
            for line in fh:
                m = re.match(r'TRAFFIC kernel="([^"]+)" class=(\S+) src=(\S+) bytes=(\d+)', line)
                if m and m.group(1) == kernel and m.group(2) == cls and m.group(3) == want:
                    return int(m.group(4))
    return None


# ---------------------------------------------------------------- helpers
def build_model(R, shape, n_slots, max_B, max_T):
    import synth
    t0 = time.time()
    w = synth.make_weights(shape)
    log(f"[bench] generated {shape.name} weights in {time.time() - t0:.1f}s")
    t0 = time.time()
    m = R.Model.from_numpy(shape, w, n_slots=n_slots, max_B=max_B, max_T=max_T)
    log(f"[bench] packed on device in {time.time() - t0:.1f}s")
    return m, w


def i32(x):
    import torch
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device="cuda")


def measure_active_fraction(R, m, B):
    import torch
    p_pre, p_mask, p_act, p_cnt = R.rwkv7_debug_cmix_buffers(m.handle, m.ws, B)
    off = p_cnt - m.ws.data_ptr()
    torch.cuda.synchronize()
    return int(m.ws[off:off + 4].view(torch.int32).item())


def kernel_breakdown(R, m, B, run_step, steps=4):
    import torch
    m.set_option(R.OPT_KERNEL_TIMING, 1)
    try:
        R.rwkv7_kernel_timing(m.handle, 0, reset=True)
        for _ in range(steps):
            run_step()
        torch.cuda.synchronize()
        out = {}
        for k, name in enumerate(R.K_NAMES):
            ms, n = R.rwkv7_kernel_timing(m.handle, k)
            out[name] = {"ms_per_step": ms / steps, "launches_per_step": n / steps}
        R.rwkv7_kernel_timing(m.handle, 0, reset=True)
    finally:
        m.set_option(R.OPT_KERNEL_TIMING, 0)
    return out


def time_repeats(run_step, steps: int, repeats: int):
    """Wall time of `steps` consecutive steps, `repeats` times, each bracketed
    by a device synchronisation on both sides; returns the list of seconds."""
    import torch
    out = []
    for _ in range(max(1, repeats)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run_step()
        torch.cuda.synchronize()
        out.append(time.perf_counter() - t0)
    return out


def hbm_attainable(R):
    """Measured streaming-read bandwidth (rwkv7_read_bandwidth: every 16-byte
    chunk once, non-temporal and plain loads) of a 4 GiB buffer, far beyond
    the 256 MB MALL: the attainable HBM read rate, reported beside the 8 TB/s
    peak that the roofline fractions use.  Also the re-read rate of a 64 MB
    buffer (plain loads), which the MALL can serve between kernels."""
    import torch
    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    small = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    res = {"read_gbs": round(R.rwkv7_read_bandwidth(big, True, 5), 1),
           "read_plain_gbs": round(R.rwkv7_read_bandwidth(big, False, 5), 1),
           "reread_64mb_gbs": round(R.rwkv7_read_bandwidth(small, False, 20), 1),
           "how": "rwkv7_read_bandwidth: 8 workgroups x 256 threads per CU, grid-stride 16-byte loads, "
                  "4 GiB buffer (5 launches after one warm-up); re-read: a 64 MB buffer, 20 launches"}
    del big, small
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- decode B=1 (headline)
def decode_b1(R, args, shape, m):
    import torch
    import synth
    wl = synth.WORKLOADS["decode_b1_2.9b"]
    p = synth.prompt_tokens(wl, 0, 64)
    slot = i32([0])
    m.reset(slot)
    m.prefill(0, i32(p[:63]))
    tok = i32([p[63]])                       # also the greedy output buffer
    logits = torch.empty(1, shape.vocab, device="cuda")
    occ = torch.zeros(m.n_slots, shape.vocab, device="cuda")
    zero = torch.zeros(1, device="cuda")
    one = torch.ones(1, device="cuda")

    def run_step():
        m.decode_step(slot, tok, logits)
        m.greedy(logits, occ, slot, zero, zero, one, tok)

    for _ in range(args.warmup):
        run_step()
    reps = time_repeats(run_step, args.steps, args.repeats)
    dt = float(np.median(reps))
    flags = m.poll_error()
    if flags:
        raise RuntimeError(f"device error flags {flags} during the timed decode")
    nnz = measure_active_fraction(R, m, 1)
    log(f"[bench] B=1: {args.steps} steps, median of {len(reps)} repeats {dt * 1e3:.1f} ms -> "
        f"{args.steps / dt:.1f} tok/s (repeats {[round(args.steps / r, 1) for r in reps]}); "
        f"last-layer active rows {nnz}/{shape.ffn}")
    kb = kernel_breakdown(R, m, 1, run_step)
    return dt, reps, nnz, kb, run_step, slot, tok, logits


def roofline_b1(R, shape, m, kb, nnz, slot, tok, logits):
    """Dominant kernel class of the B=1 step, timed in isolation with HIP events."""
    fused = bool(R.rwkv7_get_option(m.handle, R.OPT_FUSE_VALUE))
    cb = class_bytes(shape, 1, nnz, True, fused)
    dom = max((k for k in kb if k in cb and k != "other"), key=lambda k: kb[k]["ms_per_step"])
    cls = R.K_NAMES.index(dom)
    # a per-layer class is swept over all layers (as inside a step, no weight is re-read
    # by the next launch); the head has one layer
    layer, iters = (shape.n_layer, 200) if dom == "head" else (-1, 8)
    avg_ms = R.rwkv7_time_kernel(m.handle, m.pool, m.n_slots, slot, tok, logits, cls, layer, iters, m.ws)
    gbs = cb[dom] / (avg_ms * 1e-3) / 1e9
    kname = R.rwkv7_kernel_name(m.handle, cls, 1)
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": pmc_traffic(kname, dom),
            "scope": "dominant kernel (frac); step_frac below is the whole decode step",
            "kernel": kname, "class": dom,
            "bytes_per_launch": int(cb[dom]), "avg_launch_us": round(avg_ms * 1e3, 3),
            "launches_per_step": kb[dom]["launches_per_step"]}


def int8_b1(R, args, shape, m, run_step, slot, tok, logits):
    """The B=1 workload with the int8 weight route (rwkv7_quantize_int8 +
    RWKV7_OPT_INT8): the same steps, timed the same way, and its dominant
    kernel class against the HBM roofline with the int8 algorithmic bytes."""
    import torch
    buf = torch.empty(R.rwkv7_int8_bytes(m.cfg), dtype=torch.uint8, device="cuda")
    R.rwkv7_quantize_int8(m.handle, buf)
    R.rwkv7_set_option(m.handle, R.OPT_INT8, 1)
    try:
        for _ in range(args.warmup):
            run_step()
        dt = float(np.median(time_repeats(run_step, args.steps, args.repeats)))
        if m.poll_error():
            raise RuntimeError("device error flags during the int8 decode")
        nnz = measure_active_fraction(R, m, 1)
        kb = kernel_breakdown(R, m, 1, run_step)
        cb = class_bytes(shape, 1, nnz, True, True, int8=True)
        dom = max((k for k in kb if k in cb and k != "other"), key=lambda k: kb[k]["ms_per_step"])
        cls = R.K_NAMES.index(dom)
        layer, iters = (shape.n_layer, 200) if dom == "head" else (-1, 8)
        avg_ms = R.rwkv7_time_kernel(m.handle, m.pool, m.n_slots, slot, tok, logits, cls, layer, iters, m.ws)
        gbs = cb[dom] / (avg_ms * 1e-3) / 1e9
        ms = dt / args.steps * 1e3
        sb = step_bytes(shape, 1, nnz, True, int8=True)
        kname = R.rwkv7_kernel_name(m.handle, cls, 1)
    finally:
        R.rwkv7_set_option(m.handle, R.OPT_INT8, 0)
    del buf
    res = {"tok_s": round(args.steps / dt, 1), "ms_per_step": round(ms, 4), "step_bytes": int(sb),
           "step_gbs": round(sb / (ms * 1e-3) / 1e9, 1),
           "step_hbm_frac": round(sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "roofline": {"bound": "hbm", "class": dom, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": int(cb[dom]),
                        "avg_launch_us": round(avg_ms * 1e3, 3), "kernel": kname,
                        "traffic": pmc_traffic(kname, dom)},
           "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in kb.items()}}
    log(f"[bench] B=1 int8 weights: {res['tok_s']} tok/s, {ms:.3f} ms/step, step {res['step_gbs']} GB/s; "
        f"dominant {dom} {res['roofline']['achieved']} GB/s")
    return res


# ---------------------------------------------------------------- batched decode
def batched(R, args, shape, m, B):
    import torch
    import synth
    wl = synth.WORKLOADS[f"decode_b{B}_{shape.name}"]
    lens = synth.prompt_lengths(wl, B)
    if args.prompt_len > 0:        # profiling aid: same decode shapes, short prompts
        lens = np.full(B, args.prompt_len, dtype=np.int64)
    slots_l = list(range(B))
    slots = i32(slots_l)
    m.reset(slots)
    t0 = time.time()
    for b in range(B):
        pr = synth.prompt_tokens(wl, b, int(lens[b]))
        m.prefill(b, i32(pr[:-1]))
    torch.cuda.synchronize()
    t_pf = time.time() - t0
    first = i32([synth.prompt_tokens(wl, b, int(lens[b]))[-1] for b in range(B)])
    tok = first.clone()
    logits = torch.empty(B, shape.vocab, device="cuda")
    occ = torch.zeros(m.n_slots, shape.vocab, device="cuda")
    pres = torch.full((B,), wl.presence, device="cuda")
    freq = torch.full((B,), wl.frequency, device="cuda")
    dec = torch.full((B,), wl.decay, device="cuda")

    def run_step():
        m.decode_step(slots, tok, logits)
        m.greedy(logits, occ, slots, pres, freq, dec, tok)

    for _ in range(args.warmup):
        run_step()
    reps = time_repeats(run_step, args.batched_steps, args.repeats)
    dt = float(np.median(reps))
    flags = m.poll_error()
    if flags:
        raise RuntimeError(f"device error flags {flags} during batched decode B={B}")
    kb = kernel_breakdown(R, m, B, run_step, steps=2)
    sparse = B <= R.rwkv7_get_option(m.handle, R.OPT_SPARSE_MAX_B)
    sb = step_bytes(shape, B, shape.ffn, sparse)
    ms = dt / args.batched_steps * 1e3
    res = {"model": f"{shape.name}-shape", "B": B, "tok_s": round(B * args.batched_steps / dt, 1),
           "ms_per_step": round(ms, 4),
           "tok_s_repeats": [round(B * args.batched_steps / r, 1) for r in reps],
           "steps": args.batched_steps, "prefill_s": round(t_pf, 2),
           "prompt_tokens": int(lens.sum()),
           "step_gbs": round(sb / (ms * 1e-3) / 1e9, 1),
           "step_hbm_frac": round(sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in kb.items()}}
    # MFMA rate of each projection, timed in isolation
    fl = class_flops(shape, B)
    proj = {}
    for name in ("proj_in", "proj_out", "cmix_key", "cmix_value", "head"):
        cls = R.K_NAMES.index(name)
        layer, iters = (shape.n_layer, 20) if name == "head" else (-1, 1)
        avg = R.rwkv7_time_kernel(m.handle, m.pool, m.n_slots, slots, tok, logits, cls, layer, iters, m.ws)
        tf = fl[name] / (avg * 1e-3) / 1e12
        proj[name] = {"us": round(avg * 1e3, 2), "tflops": round(tf, 1),
                      "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
    res["projections"] = proj
    res["sample"] = sample_timing(R, m, logits, occ, slots, pres, freq, dec)
    log(f"[bench] B={B}: {res['tok_s']} tok/s, {ms:.3f} ms/step, step {res['step_gbs']} GB/s; "
        f"rwkv7_sample {res['sample']['us']} us")
    return res


def sample_timing(R, m, logits, occ, slots, pres, freq, dec, reps=20):
    """rwkv7_sample on a step's logits with the adapter defaults the pages give
    (temperature 1.0, top_p 0.3, top_k 0) and the workload's penalties; seeded
    uniforms, a copy of the occurrence rows.  Algorithmic bytes: logits read
    plus occurrence read and write (12 B per token); the second read of the
    logits and occurrences and the key workspace (written once, read again
    by the selection's gather) are not counted."""
    import torch
    B, V = logits.shape
    ws = torch.zeros(R.rwkv7_sample_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    occ2 = occ.clone()
    temp = torch.ones(B, device="cuda")
    top_p = torch.full((B,), 0.3, device="cuda")
    top_k = torch.zeros(B, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    uni = torch.rand(B, device="cuda", generator=g)
    ids = torch.empty(B, dtype=torch.int32, device="cuda")

    def call():
        R.rwkv7_sample(logits, occ2, m.n_slots, slots, pres, freq, dec, temp, top_p, top_k, None, uni, ids, ws)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    if R.rwkv7_poll_error(ws):
        raise RuntimeError("device error flags from rwkv7_sample")
    gbs = 12.0 * B * V / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "distinct_ids": int(torch.unique(ids).numel())}


# ---------------------------------------------------------------- serving
def serving(R, shape, m, max_b, n_tasks, new_tokens, system_len=0, use_cache=False):
    """The continuous-batching scheduler (rwkv7_sched over the GPU backend) on a
    synthetic serving load: n_tasks prompts with the decode workload's length
    mix, each generating new_tokens tokens with the adapter's sampling defaults
    (temperature 1.0, top_p 0.3, top_k 0) and the workload's penalties, at most
    max_b at once.  Wall time from the first round to the last task's end,
    prefills included; generated tokens per second of it.
    system_len > 0: every prompt is one shared system_len-token system prompt
    followed by a suffix a tenth of the mix's length; use_cache attaches a
    prefix-state cache holding the system prompt's state, stored before the
    timed region."""
    import torch
    import synth
    wl = synth.WORKLOADS[f"decode_b{max_b}_{shape.name}"]
    lens = synth.prompt_lengths(wl, n_tasks)
    if system_len:
        lens = np.maximum(lens // 10, 2)
    V = shape.vocab
    occ = torch.zeros(m.n_slots * V, device="cuda")
    sws = torch.zeros(R.rwkv7_sample_workspace_bytes(max_b, V), dtype=torch.uint8, device="cuda")
    be = R.rwkv7_sched_gpu_backend(m.handle, m.pool, m.n_slots, occ, None, max_b, m.ws, sws, m.max_T)
    system = synth.prefill_tokens(wl, system_len).tolist() if system_len else []
    cache = arena = None
    restore = None
    if use_cache:
        snap = R.rwkv7_snapshot_bytes(m.cfg)
        arena = torch.empty(4 * ((snap + 255) // 256 * 256), dtype=torch.uint8, device="cuda")
        cache = R.rwkv7_prefix_cache_create(m.handle, arena)
        m.reset(i32([0]))
        m.prefill(0, i32(system))
        R.rwkv7_prefix_cache_store(cache, m.pool, m.n_slots, 0, system)
        # restore cost: one snapshot copied into a slot (read + write of the snapshot)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        R.rwkv7_prefix_cache_lookup(cache, m.pool, m.n_slots, 1, system)
        e0.record()
        for _ in range(20):
            R.rwkv7_prefix_cache_lookup(cache, m.pool, m.n_slots, 1, system)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 20
        restore = {"snapshot_bytes": snap, "us": round(us, 2), "gbs": round(2 * snap / (us * 1e-6) / 1e9, 1)}
        R.rwkv7_sched_gpu_backend_set_cache(be, cache)
    s = R.rwkv7_sched_create(R.SchedConfig(max_b, 0, 0, 0, V), be)
    for i in range(n_tasks):
        prm = R.SchedParams(1.0, 0.3, 0, wl.presence, wl.frequency, wl.decay, new_tokens, -1, 9000 + i)
        R.rwkv7_sched_submit(s, system + synth.prompt_tokens(wl, i, int(lens[i])).tolist(), prm)
    torch.cuda.synchronize()
    rounds = rows = seq = seq_tok = gen = 0
    t0 = time.perf_counter()
    for _ in range(n_tasks * (new_tokens + int(lens.max()) + 2)):   # every round makes progress
        st = R.rwkv7_sched_step(s)
        rounds += 1
        rows += st.decode_rows + st.one_prefill_rows
        seq += st.seq_prefills
        seq_tok += st.seq_prefill_tokens
        gen += st.decode_rows
        R.rwkv7_sched_poll(s)
        if st.active == 0 and st.queued == 0:
            break
    else:
        raise RuntimeError("the scheduler did not drain its tasks")
    dt = time.perf_counter() - t0
    restored, prefilled = R.rwkv7_sched_gpu_backend_counts(be)
    R.rwkv7_sched_free(s)
    R.rwkv7_sched_gpu_backend_free(be)
    if cache:
        R.rwkv7_prefix_cache_free(cache)
    if gen != n_tasks * new_tokens:
        raise RuntimeError(f"scheduler generated {gen} tokens, expected {n_tasks * new_tokens}")
    res = {"max_batch": max_b, "tasks": n_tasks, "new_tokens": new_tokens,
           "prompt_tokens": int(lens.sum()) + n_tasks * len(system), "system_prompt": len(system),
           "prefix_cache": use_cache, "tokens_restored": restored, "tokens_prefilled": prefilled,
           "snapshot_restore": restore,
           "seconds": round(dt, 3), "gen_tok_s": round(gen / dt, 1), "rounds": rounds,
           "mean_rows_per_round": round(rows / rounds, 2), "seq_prefills": seq, "seq_prefill_tokens": seq_tok,
           "ms_per_round": round(dt / rounds * 1e3, 3)}
    log(f"[bench] scheduler max_batch={max_b} system={len(system)} cache={use_cache}: {res['gen_tok_s']} "
        f"generated tok/s over {rounds} rounds ({res['mean_rows_per_round']} rows/round, {seq} sequence "
        f"prefills, {prefilled} tokens prefilled, {restored} restored)")
    return res


# ---------------------------------------------------------------- prefill
def prefill(R, shape, m, Ts):
    import torch
    import synth
    wl = synth.WORKLOADS["prefill_2.9b"]
    out = {}
    for T in Ts:
        toks = i32(synth.prefill_tokens(wl, T))
        slot = i32([0])
        m.reset(slot)
        m.prefill(0, toks)      # warm-up
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            m.reset(slot)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            m.prefill(0, toks)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        dt = float(np.median(times))
        out[str(T)] = {"tok_s": round(T / dt, 1), "ms": round(dt * 1e3, 3)}
        log(f"[bench] prefill T={T}: {T / dt:.0f} tok/s")
    return out


# ---------------------------------------------------------------- CPU oracle
def cpu_baseline(shape, weights, seconds):
    """The fp64 oracle (oracle/rwkv7.py, unchanged) timed on the host cores on a
    bounded sample of each workload it can reach within about `seconds`:
      tiny        the whole workload (7 prompt tokens prefilled, 16 decode steps);
      2.9B B=1    decode steps (the headline `value`, tokens/s);
      2.9B B=8    batched decode steps of eight rows, the protocol subset size
                  of the B = 64 / 256 workloads (rows x steps per second);
      2.9B T=128  one 128-token sequence prefill (tokens/s).
    The oracle keeps fp64 copies of the weights (Weights(cache=True)); that
    one-time conversion is outside the timed regions, as the GPU's weight
    packing is.  States start at zero: the oracle's cost does not depend on
    their contents.  The 7.2B shape is not timed (another 58 GB of fp64
    copies on the host)."""
    from oracle import rwkv7 as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:
        blas = []
    cores = len(os.sched_getaffinity(0))
    threads = max([n for _, n in blas if n] or [1])
    per = {}

    def timed(fn, budget, max_n):
        n, t0 = 0, time.perf_counter()
        while n < max_n:
            fn(n)
            n += 1
            if time.perf_counter() - t0 >= budget:
                break
        return n, time.perf_counter() - t0

    # tiny, in full
    tw = synth.make_weights(synth.TINY)
    Wt = O.Weights(synth.TINY, tw, cache=True)
    wl = synth.WORKLOADS["tiny"]
    p = synth.prompt_tokens(wl, 0, 8)
    feeds = [int(p[7])] + [int(t) for t in synth.teacher_stream(wl, 0, 15)]
    st = O.State(synth.TINY)
    t0 = time.perf_counter()
    O.seq(Wt, st, p[:7], want_logits=False)
    t1 = time.perf_counter()
    for t in feeds:
        O.step(Wt, [st], [t])
    t2 = time.perf_counter()
    per["tiny"] = {"decode_tok_s": round(16 / (t2 - t1), 2), "total_s": round(t2 - t0, 3),
                   "sample": "7-token prefill + 16 decode steps (the whole workload)"}

    t0 = time.perf_counter()
    W = O.Weights(shape, weights, cache=True)
    for name in weights:
        W(name)
    upcast_s = time.perf_counter() - t0
    toks = synth.teacher_stream(synth.WORKLOADS["decode_b1_2.9b"], 0, 64)
    st = O.State(shape)
    n, dt = timed(lambda i: O.step(W, [st], [int(toks[i])]), 0.4 * seconds, 16)
    value = n / dt
    per["decode_b1_2.9b"] = {"tok_s": round(value, 3), "steps": n}
    states = [O.State(shape) for _ in range(8)]
    tb = synth.teacher_stream(synth.WORKLOADS["decode_b64_2.9b"], 0, 64)
    n, dt = timed(lambda i: O.step(W, states, [int(x) for x in tb[8 * i % 56: 8 * i % 56 + 8]]),
                  0.3 * seconds, 16)
    per["decode_b8_2.9b"] = {"row_tok_s": round(8 * n / dt, 3), "steps": n,
                             "sample": "8 rows per step (the protocol subset of the B=64 / B=256 workloads)"}
    pt = synth.prefill_tokens(synth.WORKLOADS["prefill_2.9b"], 128)
    st = O.State(shape)
    t0 = time.perf_counter()
    O.seq(W, st, pt, want_logits=False)
    per["prefill_2.9b_T128"] = {"tok_s": round(128 / (time.perf_counter() - t0), 3)}
    del W
    return {"value": round(value, 4), "unit": "tokens/s", "cores": int(min(threads, cores)),
            "kind": "oracle",
            "sample": f"{per['decode_b1_2.9b']['steps']} fp64 decode steps of the 2.9B-shape model, B=1 "
                      f"(value); also tiny in full, 8-row batched steps and a 128-token prefill (per_config); "
                      f"NumPy with BLAS {blas}, {cores} host cores visible; fp64 weight copies made once "
                      f"({upcast_s:.1f} s, untimed)",
            "per_config": per}


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--batched", default="64,256", help="extra batched-decode B values ('' = none)")
    ap.add_argument("--batched-steps", type=int, default=128)
    ap.add_argument("--prefill", default="128,512,2048", help="prefill T values ('' = none)")
    ap.add_argument("--big", default="256", help="batched-decode B values of the 7.2B shape ('' = none)")
    ap.add_argument("--prompt-len", type=int, default=0,
                    help="batched decode: fixed prompt length instead of the workload's 20-2000 "
                         "(profiling runs only; the decode step shapes do not change)")
    ap.add_argument("--serve", default="64", help="scheduler max_batch values ('' = none)")
    ap.add_argument("--serve-tasks", type=int, default=128)
    ap.add_argument("--serve-new", type=int, default=256)
    ap.add_argument("--serve-system", type=int, default=1024,
                    help="shared system-prompt length of the prefix-cache serving runs (0 = none)")
    ap.add_argument("--no-int8", dest="int8", action="store_false",
                    help="skip the B=1 run on int8 weights")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed passes of K steps per decode config; the median is reported")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="time budget of the CPU oracle baseline (split over its configs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Decode would shard by state slots, one process per GPU, with no communication.", file=sys.stderr)
        sys.exit(2)

    import torch
    import rwkv_linear_attention_decode_amd as R
    import synth
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible: the HIP library needs an MI355X")
    shape = synth.R7_2B9
    Bs = [int(b) for b in args.batched.split(",") if b]
    Ts = [int(t) for t in args.prefill.split(",") if t]
    Ss = [int(b) for b in args.serve.split(",") if b]
    n_slots = max([1] + Bs + Ss)
    m, weights = build_model(R, shape, n_slots=n_slots, max_B=max([1] + Bs + Ss),
                             max_T=max([512] + Ts))

    hbm = hbm_attainable(R)
    log(f"[bench] streaming read: {hbm['read_gbs']} GB/s (4 GiB, non-temporal), {hbm['read_plain_gbs']} GB/s "
        f"(plain); 64 MB re-read {hbm['reread_64mb_gbs']} GB/s")
    dt, reps, nnz, kb, run_step, slot, tok, logits = decode_b1(R, args, shape, m)
    ms = dt / args.steps * 1e3
    sb = step_bytes(shape, 1, nnz, True)
    roof = roofline_b1(R, shape, m, kb, nnz, slot, tok, logits)
    roof["step_frac"] = round(sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    log(f"[bench] dominant kernel {roof['class']}: {roof['avg_launch_us']} us/launch, "
        f"{roof['achieved']} GB/s ({roof['frac'] * 100:.1f}% of HBM peak)")
    i8 = int8_b1(R, args, shape, m, run_step, slot, tok, logits) if args.int8 else None
    pen = torch.ones(1, device="cuda")
    samp_b1 = sample_timing(R, m, logits, torch.zeros(m.n_slots, shape.vocab, device="cuda"), slot, pen, pen,
                            pen * 0.996)
    log(f"[bench] rwkv7_sample B=1: {samp_b1['us']} us")

    batched_res = [batched(R, args, shape, m, B) for B in Bs]
    prefill_res = prefill(R, shape, m, Ts) if Ts else {}
    serve_res = [serving(R, shape, m, B, args.serve_tasks, args.serve_new) for B in Ss]
    for B in Ss[:1]:
        if args.serve_system > 0:
            for use_cache in (False, True):
                serve_res.append(serving(R, shape, m, B, args.serve_tasks, args.serve_new,
                                         args.serve_system, use_cache))
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        cpu = cpu_baseline(shape, weights, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']} tok/s")
    m.close()
    del weights

    # the 7.2B shape: batched decode only (its B=1 and prefill paths are the same kernels)
    big_res = []
    Bb = [int(b) for b in args.big.split(",") if b]
    if Bb:
        torch.cuda.empty_cache()
        m7, _ = build_model(R, synth.R7_7B2, n_slots=max(Bb), max_B=max(Bb), max_T=512)
        big_res = [batched(R, args, synth.R7_7B2, m7, B) for B in Bb]
        m7.close()

    line = {
        "metric": METRIC, "value": round(args.steps / dt, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "rwkv7 2.9B-shape decode, B=1, 64-token uniform-id prompt, greedy",
                   "batch": 1, "prompt_tokens": 64, "weights": "fp16 random-init", "state": "fp32",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "repeats": {"n": len(reps), "tok_s": [round(args.steps / r, 2) for r in reps],
                    "value_is": "median"},
        "step": {"bytes": int(sb), "gbs": round(sb / (ms * 1e-3) / 1e9, 1),
                 "hbm_frac": round(sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "hbm_frac_of_measured_read": round(sb / (ms * 1e-3) / 1e9 / hbm["read_gbs"], 4),
                 "active_ffn_rows_last_layer": nnz},
        "hbm_measured": hbm,
        "kernels": {k: {"ms_per_step": round(v["ms_per_step"], 4),
                        "launches_per_step": v["launches_per_step"]} for k, v in kb.items()},
        "batched": batched_res + big_res,
        "sample_b1": samp_b1,
        "int8_b1": i8,
        "prefill": prefill_res,
        "serving": serve_res,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
