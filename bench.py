#!/usr/bin/env python3
"""Decode attention + eviction throughput on one MI355X.

Workload (default): the heavy-load layer -- batch 512, 64 query / 8 kv heads,
head_dim 128, bf16, 2,048-token prompts -- under H2O-512 (64 heavy + 448
recent).  Step 1 trims every unit from 2,049 attended tokens to 512 and is
reported on its own; the timed steps are the steady state, one whole decode
step each: attention for every sequence (new token included), the H2O score
update, the selection and the compaction, all on the GPU.

Prints one JSON line (rank 0, N = 1):
  value = decode steps/s (whole batch), roofline of the dominant kernel
  (algorithmic bytes / its HIP-event duration vs 8 TB/s), and the CPU oracle
  timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM traffic of the fused step kernel at the heavy-load shape, from two
# rocprofv3 --pmc runs of this script per case (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch, mean over the steady-state dispatches), each scaled by what the
# same counter reads for a plain 1 GiB device copy (--copy-probe-mb 1024):
# FETCH_SIZE reads 524,301.2 KiB for 1,048,576 KiB copied (x 2.000),
# WRITE_SIZE reads 1,048,576 KiB (x 1.000).  A record is valid only for the
# fused kernel's sources whose digest it holds; otherwise the bench reports null.
FETCH_SCALE = 1048576.0 / 524301.20
WRITE_SCALE = 1.0
PROFILED_TRAFFIC = [
    {"sources_digest": "c0791d2f6fa3568a", "workload": "heavy_load_b512_l2048", "policy": "h2o",
     "kv_dtype": "bf16", "fetch_kib": 538442.26, "write_kib": 26995.57},
    {"sources_digest": "c0791d2f6fa3568a", "workload": "heavy_load_b512_l2048", "policy": "streaming",
     "kv_dtype": "bf16", "fetch_kib": 534098.69, "write_kib": 18688.10},
    {"sources_digest": "c0791d2f6fa3568a", "workload": "heavy_load_b512_l2048", "policy": "h2o",
     "kv_dtype": "e5m2", "fetch_kib": 276357.07, "write_kib": 25968.04},
]


# the translation unit of the fused step kernel: its source and every header it
# includes from this repository
FUSED_SOURCES = ["compressed_decode_attention_amd/csrc/fused.hip",
                 "compressed_decode_attention_amd/csrc/mfma_tiles.h",
                 "compressed_decode_attention_amd/csrc/generic.h",
                 "compressed_decode_attention_amd/csrc/kvc_internal.h",
                 "include/kvc.h"]


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in FUSED_SOURCES:
        h.update(os.path.basename(f).encode())
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload: str, policy: str, kv_dtype: str):
    """(bytes per launch, where the figure comes from): a stored counter
    record for these exact fused-kernel sources, or (None, why not)."""
    digest = sources_digest()
    for t in PROFILED_TRAFFIC:
        if (t["workload"], t["policy"], t["kv_dtype"], t["sources_digest"]) == \
                (workload, policy, kv_dtype, digest):
            return ((t["fetch_kib"] * FETCH_SCALE + t["write_kib"] * WRITE_SCALE) * 1024.0,
                    f"stored record, not measured in this run: rocprofv3 --pmc FETCH_SIZE and "
                    f"WRITE_SIZE of this script at this workload, policy and cache dtype, "
                    f"calibrated on a 1 GiB copy, for fused-kernel sources digest {digest}")
    return None, (f"none: no counter record for the current fused-kernel sources "
                  f"(digest {digest}) at this workload, policy and cache dtype")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def per_unit_bytes(n: int, G: int, D: int, b: int, policy: str, act_b: int = 0) -> int:
    """Algorithmic HBM bytes of one unit (sequence x kv head) in one steady step.

    n = cached slots before the step, b = bytes of a cached K / V element,
    act_b = bytes of an activation element (q, k_new, v_new; default b).  K and
    V of the n cached slots are read once; the new token's k, v are read once
    (activations) and written once (cache elements); the group's q is read
    and its fp32 output written; H2O reads and writes one fp32 score per
    attended slot; every policy but 'full' reads one int32 position per cached
    slot (the selection), and the new slot's position is written.
    """
    act_b = act_b or b
    kv = 2 * n * D * b
    new = 2 * D * act_b + 2 * D * b
    qo = G * D * (act_b + 4)
    sc = 8 * (n + 1) if policy.startswith("h2o") else 0
    pos = 4 * n if policy != "full" else 0
    return kv + new + qo + sc + pos + 4


def cpu_baseline(w, n_cached: int, budget_s: float = 12.0, decay: float = 0.0,
                 policy: str = "h2o"):
    """The oracle (single thread) stepping the whole batch at the same shape
    from a steady state of n_cached entries per unit, whole decode steps until
    about budget_s seconds of work have been timed."""
    import oracle
    import synth
    import numpy as np
    orc = oracle.Oracle(w.q_heads, w.kv_heads, w.head_dim, w.dtype)
    if policy == "random":
        pol = oracle.Policy.random(w.pinned, w.n_keep, w.seed)
        pos, seen = np.arange(n_cached), n_cached
    else:
        if policy == "streaming":
            pol = oracle.Policy.streaming(w.n_sink, w.n_recent)
        elif policy == "full":
            pol = oracle.Policy.full()
        else:
            pol = oracle.Policy.h2o(w.n_heavy, w.n_recent, decay=decay)
        # steady state: the first n_sink/n_heavy positions plus the recent window
        keep = n_cached - w.n_recent
        pos = np.concatenate([np.arange(keep), np.arange(w.prompt_len - w.n_recent, w.prompt_len)])
        seen = w.prompt_len
    for b in range(w.batch):
        k, v = synth.prefill_kv(w, b, n_cached)
        orc.load(b, k, v, seen=seen, pos=[pos] * w.kv_heads)
    t_work = 0.0
    steps = 0
    while t_work < budget_s and steps < 64:
        steps += 1
        inputs = [synth.step_inputs(w, b, steps) for b in range(w.batch)]
        t0 = time.perf_counter()
        for b in range(w.batch):
            orc.step(b, *inputs[b], pol, step=steps)
        t_work += time.perf_counter() - t0
    return {
        "value": steps / t_work,
        "unit": "steps/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{steps} whole-batch {policy} steps ({w.batch} sequences x {w.kv_heads} kv heads, "
                   f"{n_cached} cached + 1 new per unit, fp64, one thread), "
                   f"{t_work:.1f} s of timed work"),
        "host_cpu": host_cpu_model(),
        "host_nproc": os.cpu_count(),
    }


def host_cpu_model() -> str:
    """The host CPU's model name as /proc/cpuinfo reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def copy_probe(torch, mib: int, reps: int = 5):
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
    counter readings calibrate the counters against exact byte counts."""
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_probe_bytes": n, "reps": reps, "ms_per_copy": ms,
                      "copy_gbs_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def attainable_read_gbs(torch, kvc, mib: int = 2048, reps: int = 10) -> dict:
    """Read-only streaming rate of this GPU: the library's streaming kernel
    reads a 2 GiB buffer once per launch (coalesced 16-byte loads over the
    whole GPU, no writes).  The nominal HBM peak stays the roofline's
    reference; this is what a plain read stream reaches on the box."""
    x = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        kvc.stream_read(x, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        kvc.stream_read(x, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = x.numel() * 4 / (ms * 1e-3) / 1e9
    del x
    return {"gbs": gbs, "how": f"kvc_stream_read over {mib} MiB, mean of {reps} launches"}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prompt_scoring(torch, kvc, synth, args):
    """H2O prompt scoring: every query row of the causal prompt (position r,
    each of the G heads of a kv head) adds its softmax probabilities over
    positions 0..r to the scores.  Algorithmic work: one QK^T over the
    visible (row, slot) pairs, 2 * D flop each (G * P * (P + 1) / 2 pairs per
    unit); the kernel's two exact passes compute the logits twice."""
    w = synth.workload(args.workload)
    B, Hq, Hkv, D, P = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.prompt_len
    G = Hq // Hkv
    dev = torch.device("cuda", 0)
    cache = kvc.KvCache(B, Hq, Hkv, D, P, kvc.BF16, device=dev)
    cache.k.copy_(synth.device_normal(cache.k.shape, w.seed, w.wid, 1,
                                      scale_rows_frac=w.heavy_frac))
    cache.pos.copy_(torch.arange(P, dtype=torch.int32, device=dev).expand(B, Hkv, P))
    cache.n_slots.fill_(P)
    q = synth.device_normal((B, P, Hq, D), w.seed, w.wid, 3)
    qp = torch.arange(P, dtype=torch.int32, device=dev).repeat(B, 1)
    scores = torch.zeros((B, Hkv, P), device=dev)
    ws = cache.prompt_workspace(P)
    stream = torch.cuda.current_stream()

    def run():
        kvc.h2o_accumulate(cache, q, P, scores, q_pos=qp, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    pairs = B * Hkv * G * P * (P + 1) // 2
    flops = 2 * D * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"prompt scoring {w.name}: {ms:.3f} ms per call, {tflops:.0f} TFLOP/s algorithmic")
    print(json.dumps({
        "metric": "H2O prompt scoring (causal prompt attention summed into the scores)",
        "value": 1e3 / ms, "unit": "calls/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "prompt": P, "causal": True},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "prompt_stats_kernel + prompt_scores_kernel",
                     "flop_per_call": flops,
                     "note": "algorithmic = one QK^T over the visible pairs; "
                             "the two exact passes compute it twice"},
    }), flush=True)


# (batch, prompt length) points of the sweep: batch at a 2,048-token prompt, then
# length at batch 64; heavy-load heads (64 q / 8 kv, head_dim 128, bf16)
SWEEP_POINTS = [(64, 2048), (128, 2048), (256, 2048), (512, 2048),
                (64, 512), (64, 1024), (64, 4096), (64, 8192)]


def sweep_point(torch, kvc, synth, B: int, P: int, policy: str, steps: int, warmup: int,
                unfused: bool = False) -> dict:
    """Steady decode steps of one (batch, prompt, policy) point.  'full' keeps
    every token (the cache grows by one per step); the others trim to 512 at
    step 1 (not timed) and then hold 512 + 1.  unfused (H2O only): attention
    without scores, then kvc_h2o_accumulate with the step's query as one row
    (a second traversal of K), then selection and compaction: the extra pass
    that a FlashAttention without exposed probabilities costs."""
    Hq, Hkv, D = 64, 8, 128
    G = Hq // Hkv
    dev = torch.device("cuda", 0)
    full = policy == "full"
    cap = P + 2 + warmup + steps if full else P + 1
    cache = kvc.KvCache(B, Hq, Hkv, D, cap, kvc.BF16, device=dev)
    for b0 in range(0, B, 64):
        sl = slice(b0, min(B, b0 + 64))
        shape = cache.k[sl, :, :P].shape
        cache.k[sl, :, :P] = synth.device_normal(shape, 0, 900 + P, 1, b0)
        cache.v[sl, :, :P] = synth.device_normal(shape, 0, 900 + P, 2, b0)
    cache.pos[:, :, :P] = torch.arange(P, dtype=torch.int32, device=dev)
    cache.n_slots.fill_(P)
    h2o = policy == "h2o"
    scores = torch.zeros((B, Hkv, cap), device=dev) if h2o else None
    pool = [(synth.device_normal((B, Hq, D), 0, 901, 3, i),
             synth.device_normal((B, Hkv, D), 0, 901, 4, i),
             synth.device_normal((B, Hkv, D), 0, 901, 5, i)) for i in range(4)]
    total = 1 + warmup + steps
    new_pos = (P + torch.arange(total, dtype=torch.int32, device=dev)).view(-1, 1).expand(
        total, B).contiguous()
    out = torch.empty((B, Hq, D), device=dev)
    pol = {"h2o": kvc.policy_h2o(64, 448), "streaming": kvc.policy_streaming(64, 448),
           "full": kvc.policy_full()}[policy]
    ws = cache.workspace(cap)
    pws = cache.prompt_workspace(1)
    keep = torch.empty((B, Hkv, cap), dtype=torch.int32, device=dev)
    nout = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    hint = [cap]

    def step(t):
        q, kn, vn = pool[t % 4]
        if unfused and t > 1:
            kvc.decode_attn(cache, new_pos[t - 1], q, kn, vn, out, None, max_len_hint=hint[0],
                            workspace=ws, stream=stream)
            kvc.h2o_accumulate(cache, q, 1, scores, workspace=pws, stream=stream)
            kvc.evict_h2o(cache, scores, 64, 448, keep, nout, stream=stream)
            kvc.compact(cache, keep, nout, scores, stream=stream)
        else:
            kvc.decode_step(cache, pol, t, new_pos[t - 1], q, kn, vn, out, scores,
                            max_len_hint=hint[0], workspace=ws, stream=stream)

    step(1)
    torch.cuda.synchronize()
    if not full:
        hint[0] = int(cache.n_slots[0, 0].item()) + 1
    for t in range(2, 2 + warmup):
        step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(2 + warmup, 2 + warmup + steps):
        step(t)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert int(cache.flags.item()) == 0
    if full:   # mean cached length over the timed steps
        n = P + 1 + warmup + (steps - 1) / 2.0
        unit = per_unit_bytes(0, G, D, 2, "full") + 2 * n * D * 2
    else:
        unit = per_unit_bytes(512, G, D, 2, policy)
    gbs = unit * B * Hkv / (ms * 1e-3) / 1e9
    del cache, scores, ws, keep
    return {"batch": B, "prompt": P, "policy": policy + ("_unfused" if unfused else ""),
            "us_per_step": ms * 1e3, "steps_per_s": 1e3 / ms, "tokens_per_s": B * 1e3 / ms,
            "algorithmic_gbs": gbs, "frac_of_8tbs": gbs / HBM_PEAK_GBS}


def kivi_unit_bytes(nq: int, nr: int, G: int, D: int = 128) -> float:
    """Algorithmic HBM bytes of one unit in one KIVI-4 decode step with nq
    quantized and nr residual tokens before the step: codes (D/2 bytes per
    token for K and for V), binary32 grids (per group 2 x D for K, per token
    2 x D/32 for V), the bf16 residual rows, the new token read (bf16) and
    written into the residual, q and the fp32 output, the two counts, and the
    conversion of 32 residual tokens every 32 steps (read 32 rows, write their
    codes and grids, move 96 rows) spread over those steps."""
    codes = nq * D                                     # K and V, 4 bits each
    grids = (nq // 32) * 2 * D * 4 + nq * 2 * (D // 32) * 4
    res = nr * 2 * D * 2
    new = 2 * D * 2 + 2 * D * 2
    qo = G * D * (2 + 4)
    conv = (32 * 2 * D * 2 + 32 * (D + 2 * D * 4 / 32 + 2 * (D // 32) * 4) + 2 * 96 * 2 * D * 2) / 32
    return codes + grids + res + new + qo + 8 + conv


def kivi_bench(torch, kvc, synth, args):
    """KIVI-4 decode steps at a workload's shape: the prompt is quantized
    (group 32, 128-token residual), then whole decode steps (attention over
    the dequantized tokens, the residual and the new token; residual
    conversion every 32 steps) are timed back to back."""
    w = synth.workload(args.workload)
    B, Hq, Hkv, D, P = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.prompt_len
    G = Hq // Hkv
    dev = torch.device("cuda", 0)
    total = 1 + args.warmup + 2 * args.steps
    mq = oracle_free_split(P + total)[0]
    cache = kvc.KiviCache(B, Hq, Hkv, D, mq, device=dev)
    k = torch.empty((B, Hkv, P, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    for b0 in range(0, B, 64):
        sl = slice(b0, min(B, b0 + 64))
        k[sl] = synth.device_normal(k[sl].shape, w.seed, w.wid, 21, b0)
        v[sl] = synth.device_normal(v[sl].shape, w.seed, w.wid, 22, b0)
    lengths = torch.full((B,), P, dtype=torch.int32, device=dev)
    kvc.kivi_prefill(cache, k, v, lengths)
    del k, v
    pool = [(synth.device_normal((B, Hq, D), w.seed, w.wid, 23, i),
             synth.device_normal((B, Hkv, D), w.seed, w.wid, 24, i),
             synth.device_normal((B, Hkv, D), w.seed, w.wid, 25, i)) for i in range(4)]
    out = torch.empty((B, Hq, D), device=dev)
    ws = cache.workspace(mq)
    stream = torch.cuda.current_stream()

    def step(t):
        q, kn, vn = pool[t % 4]
        kvc.kivi_decode(cache, q, kn, vn, out, max_quant_hint=mq, workspace=ws, stream=stream)

    t = 1
    for _ in range(args.warmup):
        step(t)
        t += 1
    torch.cuda.synchronize()
    t_first = t
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step(t)
        t += 1
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(t)
        evs[i][1].record(stream)
        t += 1
    torch.cuda.synchronize()
    launch_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    assert int(cache.flags.item()) == 0, "device contract flag raised"
    # mean algorithmic bytes over the event-bracketed steps (counts follow the
    # schedule: N tokens before a step -> kivi_split(N))
    n0 = P + (t_first - 1) + args.steps
    unit = sum(kivi_unit_bytes(*oracle_free_split(n0 + i), G, D) for i in range(args.steps)) / args.steps
    step_bytes = unit * B * Hkv
    achieved = step_bytes / (launch_ms * 1e-3) / 1e9
    attain = attainable_read_gbs(torch, kvc)
    log(f"KIVI-4 {w.name}: {ms * 1e3:.1f} us/step back to back, {launch_ms * 1e3:.1f} us per "
        f"event-bracketed step, {achieved:.0f} GB/s algorithmic")
    print(json.dumps({
        "metric": f"KIVI-4 decode steps/s and achieved HBM GB/s, B={B} L={P}",
        "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + "_kivi4", "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "prompt": P, "group": 32, "residual": 128, "bits": 4,
                   "tokens_per_s": B * 1e3 / ms},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "kvc_kivi_decode (whole step; one launch at one share per "
                               "unit: quantized tokens, residual and new token, output, "
                               "conversion, append)",
                     "bytes_per_unit": unit, "units_per_launch": B * Hkv, "launch_ms": launch_ms,
                     "attainable_read_gbs": attain["gbs"],
                     "frac_of_attainable": achieved / attain["gbs"]},
    }), flush=True)


def oracle_free_split(n_tokens: int, group: int = 32, residual: int = 128):
    """(quantized, residual) token counts of a KIVI cache holding n_tokens
    (the schedule kvc.h states; used only to size and count bytes)."""
    over = max(n_tokens - residual, 0)
    q = group * ((over + group - 1) // group)
    return q, n_tokens - q


def warm_first_step(torch, kvc, cache, pol, with_scores):
    """One untimed whole step on a one-sequence scratch cache of the same
    shape, capacity and layout, so that the timed first step does not include
    loading the long-unit kernels' code on their first launch."""
    dev = cache.k.device
    cap, bs = cache.capacity, cache.block_size
    table = torch.arange(cap // bs, dtype=torch.int32).view(1, -1) if bs else None
    s = kvc.KvCache(1, cache.q_heads, cache.kv_heads, cache.head_dim, cap, cache.dtype, device=dev,
                    block_size=bs, num_blocks=cap // bs if bs else 0, block_table=table)
    s.pos.copy_(torch.arange(cap, dtype=torch.int32, device=dev).expand(1, cache.kv_heads, cap))
    s.n_slots.fill_(cap - 1)
    act = torch.bfloat16
    q = torch.zeros((1, cache.q_heads, cache.head_dim), dtype=act, device=dev)
    kn = torch.zeros((1, cache.kv_heads, cache.head_dim), dtype=act, device=dev)
    out = torch.empty((1, cache.q_heads, cache.head_dim), device=dev)
    sc = torch.zeros((1, cache.kv_heads, cap), device=dev) if with_scores else None
    kvc.decode_step(s, pol, 1, torch.full((1,), cap - 1, dtype=torch.int32, device=dev), q, kn, kn,
                    out, sc, max_len_hint=cap, workspace=s.workspace(cap))
    torch.cuda.synchronize()
    del s



def time_one_call(torch, kvc, stream, call):
    """(GPU ms, host ms) of one call that is timed alone (the first step).
    From an idle GPU, events around the call would also bracket the host's
    argument checks and the launch of its first kernel (0.1 ms or more),
    which the back-to-back steps overlap with the previous step's kernels.
    So the call's launches are issued while the GPU still reads a 1 GiB
    buffer (the library's streaming kernel, about 0.16 ms of GPU work queued
    just before the first event): the events then bracket the call's
    kernels.  The host ms is the wall time of the call itself (enqueueing)."""
    x = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    kvc.stream_read(x, sink, stream=stream)
    e0.record(stream)
    h0 = time.perf_counter()
    call()
    h1 = time.perf_counter()
    e1.record(stream)
    torch.cuda.synchronize()
    del x
    return e0.elapsed_time(e1), (h1 - h0) * 1e3

def paged_bench(torch, kvc, synth, args, w):
    """H2O-512 on a paged cache of mixed-length sequences (log-uniform
    512..32,768 tokens, blocks of 16 slots, a shuffled block table): the first
    step (attention over every prompt, then the trim to 512) is timed alone,
    then whole steady steps back to back (one launch each)."""
    import numpy as np
    B, Hq, Hkv, D, bs = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.paged_block
    G = Hq // Hkv
    dev = torch.device("cuda", 0)
    lengths = synth.mixed_lengths(w)
    cap = (int(lengths.max()) + 1 + bs - 1) // bs * bs
    max_blocks = cap // bs
    nblk = B * max_blocks
    perm = synth.block_permutation(nblk, w.seed, w.wid, 0)
    table = torch.from_numpy(perm.reshape(B, max_blocks).copy())
    cache = kvc.KvCache(B, Hq, Hkv, D, cap, kvc.BF16, device=dev, block_size=bs, num_blocks=nblk,
                        block_table=table)
    step_blocks = 4096
    for i0 in range(0, nblk, step_blocks):
        sl = slice(i0, min(nblk, i0 + step_blocks))
        cache.k[sl] = synth.device_normal(cache.k[sl].shape, w.seed, w.wid, 31, i0)
        cache.v[sl] = synth.device_normal(cache.v[sl].shape, w.seed, w.wid, 32, i0)
    cache.pos.copy_(torch.arange(cap, dtype=torch.int32, device=dev).expand(B, Hkv, cap))
    cache.n_slots.copy_(torch.from_numpy(lengths.astype(np.int32)).view(B, 1).expand(B, Hkv))
    scores = torch.zeros((B, Hkv, cap), device=dev)
    pool = [(synth.device_normal((B, Hq, D), w.seed, w.wid, 33, i),
             synth.device_normal((B, Hkv, D), w.seed, w.wid, 34, i),
             synth.device_normal((B, Hkv, D), w.seed, w.wid, 35, i)) for i in range(4)]
    total = 1 + args.warmup + 2 * args.steps
    lens = torch.from_numpy(lengths.astype(np.int32)).to(dev)
    new_pos = (lens.view(1, B) + torch.arange(total, dtype=torch.int32, device=dev).view(-1, 1)).contiguous()
    out = torch.empty((B, Hq, D), device=dev)
    pol = kvc.policy_h2o(w.n_heavy, w.n_recent)
    ws = cache.workspace(cap)
    stream = torch.cuda.current_stream()
    hint = [cap]

    def step(t):
        q, kn, vn = pool[t % 4]
        kvc.decode_step(cache, pol, t, new_pos[t - 1], q, kn, vn, out, scores,
                        max_len_hint=hint[0], workspace=ws, stream=stream)

    warm_first_step(torch, kvc, cache, pol, True)
    trim_ms, trim_host_ms = time_one_call(torch, kvc, stream, lambda: step(1))
    assert bool((cache.n_slots == 512).all())
    hint[0] = 513
    t = 2
    for _ in range(args.warmup):
        step(t)
        t += 1
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step(t)
        t += 1
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(t)
        evs[i][1].record(stream)
        t += 1
    torch.cuda.synchronize()
    launch_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    assert int(cache.flags.item()) == 0, "device contract flag raised"
    unit = per_unit_bytes(512, G, D, 2, "h2o")
    achieved = unit * B * Hkv / (launch_ms * 1e-3) / 1e9
    first_bytes = sum(per_unit_bytes(int(L), G, D, 2, "h2o") for L in lengths) * Hkv
    log(f"{w.name}: first step {trim_ms:.3f} ms on the GPU ({first_bytes / (trim_ms * 1e-3) / 1e9:.0f} "
        f"GB/s for the attention's bytes, trim included; the call's host side {trim_host_ms:.3f} ms), "
        f"steady {ms * 1e3:.1f} us/step, {achieved:.0f} GB/s")
    print(json.dumps({
        "metric": f"decode steps/s and achieved HBM GB/s, paged mixed lengths, B={B}",
        "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "block": bs, "lengths": f"log-uniform {w.min_len}..{w.max_len}, "
                                           f"mean {float(lengths.mean()):.0f}",
                   "policy": "h2o", "budget": "64+448", "first_step_ms": trim_ms,
                   "first_step_host_ms": trim_host_ms,
                   "tokens_per_s": B * 1e3 / ms},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "kvc_decode_step (whole step, paged)", "bytes_per_unit": unit,
                     "units_per_launch": B * Hkv, "launch_ms": launch_ms},
    }), flush=True)


def whole_run(torch, kvc, synth, args):
    """Per-head random eviction over the reasoning trace's whole schedule:
    the pinned prompt, then one decode step per generated token; the cache
    grows from the prompt to the budget (pinned + n_keep, no eviction), then
    every step evicts one generated token per head.  Every step is one
    kvc_decode_step; the two phases are timed with events on the launch
    stream and the run's average is the value."""
    w = synth.workload(args.workload)
    assert w.policy == "random", "--whole-run follows a random-eviction workload's schedule"
    B, Hq, Hkv, D, P = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.pinned
    G = Hq // Hkv
    steps = w.steps
    cap = w.pinned + w.n_keep + 1
    dev = torch.device("cuda", 0)
    cache = kvc.KvCache(B, Hq, Hkv, D, cap, kvc.BF16, device=dev)
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    cache.k[:, :, :P] = torch.randn(cache.k[:, :, :P].shape, generator=gen, device=dev).to(torch.bfloat16)
    cache.v[:, :, :P] = torch.randn(cache.v[:, :, :P].shape, generator=gen, device=dev).to(torch.bfloat16)
    cache.pos[:, :, :P] = torch.arange(P, dtype=torch.int32, device=dev)
    cache.n_slots.fill_(P)
    pool = [(torch.randn((B, Hq, D), generator=gen, device=dev).to(torch.bfloat16),
             torch.randn((B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16),
             torch.randn((B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16))
            for _ in range(4)]
    new_pos = (P + torch.arange(steps, dtype=torch.int32, device=dev)).view(-1, 1).expand(
        steps, B).contiguous()
    out = torch.empty((B, Hq, D), device=dev)
    pol = kvc.policy_random(w.pinned, w.n_keep, w.seed)
    ws = cache.workspace(cap)
    stream = torch.cuda.current_stream()
    warm_first_step(torch, kvc, cache, pol, False)
    grow = w.n_keep   # steps 1 .. n_keep fill the budget; later steps evict one
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for t in range(1, steps + 1):
        if t == grow + 1:
            ev[1].record(stream)
        q, kn, vn = pool[t % 4]
        kvc.decode_step(cache, pol, t, new_pos[t - 1], q, kn, vn, out, max_len_hint=cap,
                        workspace=ws, stream=stream)
    ev[2].record(stream)
    torch.cuda.synchronize()
    assert int(cache.flags.item()) == 0, "device contract flag raised"
    assert bool((cache.n_slots == cap - 1).all())
    grow_ms, steady_ms = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    total_ms = grow_ms + steady_ms
    # algorithmic bytes: every step attends its n cached slots + the new token
    n_of = lambda t: min(P + t - 1, cap - 1)
    grow_bytes = sum(per_unit_bytes(n_of(t), G, D, 2, "random") for t in range(1, grow + 1)) * B * Hkv
    steady_bytes = per_unit_bytes(cap - 1, G, D, 2, "random") * (steps - grow) * B * Hkv
    run_gbs = (grow_bytes + steady_bytes) / (total_ms * 1e-3) / 1e9
    log(f"{w.name} whole run: {steps} steps in {total_ms:.1f} ms (growth {grow} steps "
        f"{grow_ms:.1f} ms, steady {steps - grow} steps {steady_ms:.1f} ms), {run_gbs:.0f} GB/s")
    print(json.dumps({
        "metric": f"decode steps/s over the whole random-eviction run, B={B}",
        "value": steps / (total_ms * 1e-3), "unit": "steps/s", "n_gpus": 1, "steps": steps,
        "warmup": 0, "ms_per_step": total_ms / steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "pinned": P, "n_keep": w.n_keep, "policy": "random",
                   "growth_steps": grow, "growth_us_per_step": grow_ms * 1e3 / grow,
                   "steady_steps": steps - grow,
                   "steady_us_per_step": steady_ms * 1e3 / (steps - grow),
                   "tokens_per_s": B * steps / (total_ms * 1e-3)},
        "roofline": {"bound": "hbm", "achieved": run_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": run_gbs / HBM_PEAK_GBS, "traffic": None,
                     "traffic_source": "none: not profiled for this run",
                     "kernel": "kvc_decode_step (split path: split_kernel + finish_kernel)",
                     "bytes_per_run": grow_bytes + steady_bytes},
    }), flush=True)


def cpu_baselines(args):
    """The oracle (one host thread, fp64, unmodified) on every workload's
    whole batch, a few steps each, in the phases the workload runs: one JSON
    line per (workload, phase).  No GPU is used."""
    import numpy as np
    import oracle
    import synth

    def timed(w, pol, loads, steps, first_step=1):
        orc = oracle.Oracle(w.q_heads, w.kv_heads, w.head_dim, w.dtype)
        t0 = time.perf_counter()
        for b, (n, pos, seen) in enumerate(loads):
            k, v = synth.prefill_kv(w, b, n)
            orc.load(b, k, v, seen=seen, pos=None if pos is None else [pos] * w.kv_heads)
        load_s = time.perf_counter() - t0
        work = 0.0
        for t in range(first_step, first_step + steps):
            inputs = [synth.step_inputs(w, b, t) for b in range(len(loads))]
            t1 = time.perf_counter()
            for b in range(len(loads)):
                orc.step(b, *inputs[b], pol, step=t)
            work += time.perf_counter() - t1
        return work, load_s

    def report(w, phase, pol_name, steps, work, cached):
        units = w.batch * w.kv_heads
        print(json.dumps({
            "cpu_oracle": w.name, "phase": phase, "policy": pol_name, "batch": w.batch,
            "units": units, "cached_per_unit": cached, "steps_timed": steps,
            "seconds": work, "steps_per_s": steps / work, "tokens_per_s": w.batch * steps / work,
            "cores": 1, "host_cpu": host_cpu_model(), "host_nproc": os.cpu_count(),
            "numpy": np.__version__}), flush=True)
        log(f"{w.name} {phase}: {steps / work:.4f} steps/s over {steps} steps ({work:.1f} s)")

    # tiny StreamingLLM layer: all 16 steps from 1,024 cached tokens (step 1 trims to 512)
    w = synth.workload("tiny_mha_streaming_f32")
    pol = oracle.Policy.streaming(w.n_sink, w.n_recent)
    work, _ = timed(w, pol, [(w.prompt_len, None, w.prompt_len)], w.steps)
    report(w, "all 16 steps", "streaming", w.steps, work, "1024 -> 512")

    def steady_pos(w):
        keep = 512 - w.n_recent
        return np.concatenate([np.arange(keep), np.arange(w.prompt_len - w.n_recent, w.prompt_len)])

    # H2O layers: the over-budget first step, then steady steps at 512 + 1
    for name, steady in (("llama3_8b_h2o_b64", 3), ("heavy_load_b512_l2048", 3)):
        w = synth.workload(name)
        pol = oracle.Policy.h2o(w.n_heavy, w.n_recent)
        work, _ = timed(w, pol, [(w.prompt_len, None, w.prompt_len)] * w.batch, 1)
        report(w, "step 1 (trim 2,049 -> 512)", "h2o", 1, work, w.prompt_len)
        work, _ = timed(w, pol, [(512, steady_pos(w), w.prompt_len)] * w.batch, steady, 2)
        report(w, "steady", "h2o", steady, work, 512)

    # reasoning trace, random eviction: a growth step and steady steps
    w = synth.workload("reasoning_random_b32")
    pol = oracle.Policy.random(w.pinned, w.n_keep, w.seed)
    work, _ = timed(w, pol, [(w.pinned, None, w.pinned)] * w.batch, 3)
    report(w, "growth (first steps after the 1,024-token prompt)", "random", 3, work, w.pinned)
    fill = w.pinned + w.n_keep
    work, _ = timed(w, pol, [(fill, None, fill)] * w.batch, 3, w.n_keep + 1)
    report(w, "steady (5,120 cached, one eviction per head)", "random", 3, work, fill)

    # mixed-length batch: the first step over every prompt, then steady steps
    w = synth.workload("mixed_paged_h2o_b128")
    lengths = [int(x) for x in synth.mixed_lengths(w)]
    pol = oracle.Policy.h2o(w.n_heavy, w.n_recent)
    work, _ = timed(w, pol, [(L, None, L) for L in lengths], 1)
    report(w, "step 1 (every prompt, trim to 512)", "h2o", 1, work,
           f"log-uniform 512..32768, mean {sum(lengths) / len(lengths):.0f}")
    loads = []
    for L in lengths:
        keep = 512 - w.n_recent
        loads.append((512, np.concatenate([np.arange(keep), np.arange(L - w.n_recent, L)]), L))
    work, _ = timed(w, pol, loads, 3, 2)
    report(w, "steady", "h2o", 3, work, 512)


def sweep(torch, kvc, synth, args):
    """Where eviction pays: full vs StreamingLLM-512 vs H2O-512 (and H2O with an
    unfused score pass) over batch and prompt length.  One JSON line per point."""
    Hq, Hkv, D = 64, 8, 128
    G = Hq // Hkv
    for B, P in SWEEP_POINTS:
        fused_us = None
        for policy, unfused in (("full", False), ("streaming", False), ("h2o", False),
                                ("h2o", True)):
            r = sweep_point(torch, kvc, synth, B, P, policy, args.steps, args.warmup, unfused)
            if policy == "h2o" and not unfused:
                fused_us = r["us_per_step"]
            if unfused and fused_us is not None:
                # what the unfused step would take if its second pass were
                # bandwidth-bound like the fused step: that pass's algorithmic
                # bytes (K of the 513 attended slots once, the query, the
                # scores read and written) at the fused step's achieved rate
                n = 513
                second = n * D * 2 + G * D * 2 + 8 * n
                ideal = fused_us * (1.0 + second / per_unit_bytes(512, G, D, 2, "h2o"))
                r["unfused_ideal_us_per_step"] = ideal
                r["fusion_gain_vs_measured_unfused"] = r["us_per_step"] / fused_us
                r["fusion_gain_vs_ideal_unfused"] = ideal / fused_us
            log(f"B={B} P={P} {r['policy']}: {r['us_per_step']:.1f} us/step, "
                f"{r['algorithmic_gbs']:.0f} GB/s")
            print(json.dumps(r), flush=True)
            torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="heavy_load_b512_l2048")
    ap.add_argument("--policy", default="h2o",
                    choices=["h2o", "h2o_decay", "streaming", "full", "random"],
                    help="h2o_decay: H2O with a decayed attention activity (decay 0.99); "
                         "random: per-head random eviction from a cache filled to its budget "
                         "(pinned prompt + n_keep, e.g. --workload reasoning_random_b32)")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="fp8: K / V cached as E5M2 codes (activations stay bf16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--prompt-scoring", action="store_true",
                    help="time H2O prompt scoring (kvc_h2o_accumulate over the causal prompt) "
                         "instead of the decode step")
    ap.add_argument("--sweep", action="store_true",
                    help="full / StreamingLLM / H2O (fused and unfused) over batch and prompt "
                         "length; one JSON line per point")
    ap.add_argument("--kivi", action="store_true",
                    help="KIVI-4 quantized-cache decode steps at the workload's shape")
    ap.add_argument("--whole-run", action="store_true",
                    help="random eviction over the workload's whole schedule (growth to the "
                         "budget, then one eviction per head per step; --workload "
                         "reasoning_random_b32): run-average steps/s")
    ap.add_argument("--cpu-baselines", action="store_true",
                    help="only time the CPU oracle (one thread) on every workload's phases; "
                         "no GPU")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1. "
                                   "Units (sequence, kv head) are independent, so the path "
                                   "shards by sequences or kv heads with no exchange."}))
        sys.exit(2)

    if args.cpu_baselines:
        cpu_baselines(args)
        return

    import torch

    if args.copy_probe_mb:
        copy_probe(torch, args.copy_probe_mb)
        return

    import compressed_decode_attention_amd as kvc
    import synth

    if args.prompt_scoring:
        prompt_scoring(torch, kvc, synth, args)
        return
    if args.sweep:
        sweep(torch, kvc, synth, args)
        return
    if args.kivi:
        kivi_bench(torch, kvc, synth, args)
        return
    if args.whole_run:
        whole_run(torch, kvc, synth, args)
        return

    f8 = args.kv_dtype == "fp8"
    w = synth.workload(args.workload, dtype="e5m2" if f8 else "bf16")
    if w.paged_block:
        paged_bench(torch, kvc, synth, args, w)
        return
    policy = args.policy
    B, Hq, Hkv, D, P = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.prompt_len
    if policy == "random":   # filled to the budget: every step evicts one per head
        P = w.pinned + w.n_keep
    G = Hq // Hkv
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cap = P + 1 if policy != "full" else P + 2 + args.warmup + 2 * args.steps
    log(f"workload {w.name}: B={B} Hq={Hq} Hkv={Hkv} D={D} prompt={P} policy={policy} cap={cap} "
        f"kv={w.dtype}")

    gen = torch.Generator(device=dev).manual_seed(w.seed)
    cache = kvc.KvCache(B, Hq, Hkv, D, cap, kvc.FP8_E5M2 if f8 else kvc.BF16, device=dev)

    def stored(x):
        """normal draws -> cache storage (E5M2: the draw's sign, exponent and
        top two mantissa bits; |x| < 2^-14 -> zero)"""
        if not f8:
            return x.to(torch.bfloat16)
        u = x.view(torch.int32)
        sign = (u >> 24) & 0x80
        e = (u >> 23) & 0xFF
        code = torch.where(e < 113, torch.zeros_like(u), ((e - 112) << 2) | ((u >> 21) & 3))
        return (sign | code).to(torch.uint8)

    for b0 in range(0, B, 64):
        sl = slice(b0, min(B, b0 + 64))
        cache.k[sl, :, :P] = stored(torch.randn(cache.k[sl, :, :P].shape, generator=gen,
                                                device=dev, dtype=torch.float32))
        cache.v[sl, :, :P] = stored(torch.randn(cache.v[sl, :, :P].shape, generator=gen,
                                                device=dev, dtype=torch.float32))
    cache.pos[:, :, :P] = torch.arange(P, dtype=torch.int32, device=dev)
    cache.n_slots.fill_(P)
    scores = torch.zeros((B, Hkv, cap), device=dev) if policy.startswith("h2o") else None
    n_pool = 4
    pool = [(torch.randn((B, Hq, D), generator=gen, device=dev).to(torch.bfloat16),
             torch.randn((B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16),
             torch.randn((B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16))
            for _ in range(n_pool)]
    total_steps = 1 + args.warmup + 2 * args.steps
    new_pos = (P + torch.arange(total_steps, dtype=torch.int32, device=dev)).view(-1, 1).expand(
        total_steps, B).contiguous()
    out = torch.empty((B, Hq, D), device=dev)
    if policy == "h2o":
        pol = kvc.policy_h2o(w.n_heavy, w.n_recent)
    elif policy == "h2o_decay":
        pol = kvc.policy_h2o(w.n_heavy, w.n_recent, decay=0.99)
    elif policy == "streaming":
        pol = kvc.policy_streaming(w.n_sink, w.n_recent)
    elif policy == "random":
        pol = kvc.policy_random(w.pinned, w.n_keep, w.seed)
    else:
        pol = kvc.policy_full()
    # workspace sized for the longest attended length (the first step)
    ws = cache.workspace(cap)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    # length bound passed with each step: the first step attends the whole
    # prompt; afterwards every unit holds the 512-slot budget plus the new token
    hint = [cap]

    def step(t):
        q, kn, vn = pool[t % n_pool]
        kvc.decode_step(cache, pol, t, new_pos[t - 1], q, kn, vn, out, scores,
                        max_len_hint=hint[0], workspace=ws, stream=stream)

    # step 1: the over-budget trim, timed alone (after an untimed step of the
    # same shape on a scratch cache, which loads the long-unit kernels)
    warm_first_step(torch, kvc, cache, pol, scores is not None)
    trim_ms, trim_host_ms = time_one_call(torch, kvc, stream, lambda: step(1))
    n_after = int(cache.n_slots[0, 0].item())
    log(f"step 1 (trim to {n_after}): {trim_ms:.3f} ms on the GPU (the call's host side "
        f"{trim_host_ms:.3f} ms)")
    if policy != "full":
        assert bool((cache.n_slots == n_after).all())
        hint[0] = n_after + 1

    t = 2
    for _ in range(args.warmup):
        step(t)
        t += 1
    torch.cuda.synchronize()

    # timed region: K whole steps, no host sync inside
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step(t)
        t += 1
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {total_ms:.3f} ms ({ms_per_step * 1e3:.1f} us/step), "
        f"wall {wall * 1e3:.1f} ms")

    # per-launch duration of the step, bracketed by events on the same stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(t)
        evs[i][1].record(stream)
        t += 1
    torch.cuda.synchronize()
    launch_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    assert int(cache.flags.item()) == 0, "device contract flag raised"

    attain = attainable_read_gbs(torch, kvc)
    log(f"attainable read-only stream: {attain['gbs']:.0f} GB/s")

    n_cached = n_after if policy != "full" else P + 1 + args.warmup + args.steps
    unit_bytes = per_unit_bytes(n_cached, G, D, 1 if f8 else 2, policy, act_b=2)
    step_bytes = unit_bytes * B * Hkv
    achieved = step_bytes / (launch_ms * 1e-3) / 1e9
    steps_per_s = 1e3 / ms_per_step
    traffic, traffic_source = profiled_traffic(w.name, policy, "e5m2" if f8 else "bf16")

    result = {
        "metric": f"decode steps/s and achieved HBM GB/s (% of peak), attn+evict, B={B} L={P}",
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
            "prompt": P, "policy": policy,
            "budget": {"full": "none", "random": f"{w.pinned} pinned + {w.n_keep}"}.get(policy,
                                                                                    "64+448"),
            "cached_per_unit": n_cached, "kv_dtype": "e5m2" if f8 else "bf16",
            "accumulate": "fp32",
            "tokens_per_s": steps_per_s * B, "trim_step_ms": trim_ms,
            "trim_step_host_ms": trim_host_ms,
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "traffic_source": traffic_source,
            "kernel": "kvc_decode_step (whole step)",
            "bytes_per_unit": unit_bytes, "units_per_launch": B * Hkv,
            "launch_ms": launch_ms,
            "attainable_read_gbs": attain["gbs"], "attainable_how": attain["how"],
            "frac_of_attainable": achieved / attain["gbs"],
            # the counted bytes (traffic) over the same launch time
            "counter_gbs": None if traffic is None else traffic / (launch_ms * 1e-3) / 1e9,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(
            w, n_cached if policy != "full" else P, args.cpu_budget,
            decay=0.99 if policy == "h2o_decay" else 0.0,
            policy="h2o" if policy.startswith("h2o") else policy)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
