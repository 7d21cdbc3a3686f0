#!/usr/bin/env python3
"""Benchmark of absorbed MLA decode on one MI355X.

One step = one decode call for every sequence of the workload: absorb the
queries, split-KV attention over the latent cache, fixed-order split merge and
the W_UV up-projection, i.e. the whole hot path on one batch of synthetic
input already resident in HBM.  The default workload is the DeepSeek-V3
shape at 128k context: batch 8, 128 heads, 512 + 64 latent/RoPE cache,
131072 cached tokens per sequence (bf16, fp32 accumulation).

Prints ONE JSON line: tokens/s (one new token per sequence per step), the
whole-call HBM rate against 8 TB/s, the attention kernel's own roofline
fraction from HIP events recorded around it, and the fp64 CPU oracle timed on
a bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published peak
METRIC = "decode tokens/s and achieved HBM GB/s (% of peak), MLA V3 shape @128k ctx"


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)
STEADY_SETTLE = 300  # untimed calls before the steady-state pass (decode mode)


class HipEvents:
    """hipEvent_t handles created through the HIP runtime that torch loaded,
    for timing only: without the system-scope fence (an L2 write-back and
    invalidate) that a default event performs when it is recorded, which
    leaves the GPU idle for about 6 us between the kernels it separates."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def group(self, i, k):
        arr = (ctypes.c_void_p * k)(*[self.ev[i + j].value for j in range(k)])
        return arr

    def around_attention(self, i):
        """mla_decode_profiled's four slots with events i, i + 1 around the
        split-KV kernel only (NULL slots are not recorded)."""
        return (ctypes.c_void_p * 4)(None, self.ev[i].value, self.ev[i + 1].value, None)

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "decode_splitkv_bf16_V3_B8_L131072_hbm_traffic.txt")


def measured_traffic(workload_is_profiled: bool):
    """HBM bytes per launch of the split-KV kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (copy-calibrated), or None when the kernel
    source has changed since they were taken or the workload differs."""
    import hashlib

    if not workload_is_profiled or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        kv[k.strip()] = v.strip()
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), kv.get("kernel_source", ""))
    if not os.path.isfile(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("kernel_source_sha256"):
        return None
    return float(kv["traffic_bytes_per_launch"])


def cpu_baseline(case, seconds: float):
    """fp64 oracle (absorbed form) on a bounded sample of (sequence, head) pairs
    of the same workload, all host threads; scaled to tokens/s of a full step."""
    import numpy as np

    import oracle  # test infrastructure, used here only for the CPU baseline leg
    threads = oracle.max_threads()
    rng = np.random.default_rng(123)
    total_pairs = case.B * case.H

    def sample(n):
        return [(i % case.B, int(rng.integers(case.H))) for i in range(n)]

    n0 = threads
    t = time.perf_counter()
    oracle.decode_absorbed(case.q_nope, case.q_rope, case.w_uk, case.w_uv, case.ckv, case.kpe,
                           case.seqlens, case.scale, pairs=sample(n0))
    t0 = time.perf_counter() - t
    n = int(min(total_pairs, max(n0, round(n0 * seconds / max(t0, 1e-3)))))
    # when the whole step is cheaper than the budget, it is repeated (about
    # `seconds` of CPU work in total) and the mean is reported
    reps, ts = 0, 0.0
    while reps == 0 or ts < 0.8 * seconds:
        t = time.perf_counter()
        oracle.decode_absorbed(case.q_nope, case.q_rope, case.w_uk, case.w_uv, case.ckv,
                               case.kpe, case.seqlens, case.scale, pairs=sample(n))
        ts += time.perf_counter() - t
        reps += 1
        if n < total_pairs:
            break
    t_step = ts / reps * total_pairs / n
    what = (f"{n} of {total_pairs} (sequence, head) pairs of the same workload"
            if n < total_pairs else f"the full step ({total_pairs} (sequence, head) pairs)")
    return {"value": case.B / t_step, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, {reps} pass(es), {ts:.1f} s in total, {t_step:.1f} s per step"}


def timed_back_to_back(step, steps: int) -> float:
    """Mean ms per call of `steps` calls launched back to back between one
    event pair (an event recorded between two launches idles the GPU for
    about 6 us while its timestamp is written)."""
    import torch
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def cpu_baseline_sampled(run, units, seconds: float, value_of_time, unit: str, label: str):
    """fp64 oracle on an evenly spaced sample of the call's independent units
    (query rows, sequences), all host threads: about `seconds` of host work
    (at least one unit; the whole call, repeated, when it is cheaper), scaled
    to the whole call and reported as value_of_time(seconds per call)."""
    import oracle  # test infrastructure, used here only for the CPU baseline leg
    threads = oracle.max_threads()
    n_all = len(units)

    def pick(n):
        return [units[int((i + 0.5) * n_all / n)] for i in range(n)]

    t = time.perf_counter()
    run(pick(1))
    t1 = time.perf_counter() - t
    n = int(min(n_all, max(1, round(seconds / max(t1, 1e-3)))))
    reps, ts = 0, 0.0
    while reps == 0 or (n == n_all and ts < 0.8 * seconds):
        t = time.perf_counter()
        run(pick(n))
        ts += time.perf_counter() - t
        reps += 1
    t_call = ts / reps * n_all / n
    what = (f"{n} of {n_all} {label}, evenly spaced" if n < n_all
            else f"the whole call ({n_all} {label})")
    return {"value": value_of_time(t_call), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{what}, {reps} pass(es), {ts:.1f} s in total, {t_call:.3g} s per call"}


def bench_prefill(args, mla, datagen):
    """Naive causal prefill (decompress K/V for every cached row, then causal
    attention) on the V3 shape, batch 1, 4096 tokens; one JSON line with the
    whole call's bf16 MFMA throughput against the dense peak."""
    import numpy as np
    import torch

    from mla_latent_kv_12_amd.tensors import to_device

    def latents_fp64(x, w_dkv):
        # c = W_DKV x: the prefill workload's input latents (an untimed harness
        # step, accumulated in fp64 and then stored as bf16)
        xf = datagen.bf16_to_f32(x).astype(np.float64)
        wf = datagen.bf16_to_f32(w_dkv).astype(np.float64)
        return xf @ wf.T

    case = datagen.make_workload("v3-prefill-4k", latents=latents_fp64)
    dt = case.dtype
    cache = to_device(case.cache, dt)
    q_nope, q_rope = to_device(case.q_nope, dt), to_device(case.q_rope, dt)
    w_uk, w_uv = to_device(case.w_uk, dt), to_device(case.w_uv, dt)
    ckv, kpe = cache[:, :, : case.dc], cache[:, :, case.dc:]
    seqlens = torch.from_numpy(case.seqlens.astype(np.int32)).cuda()
    params = mla.prefill_params(q_nope, q_rope, w_uk, w_uv, ckv, kpe, softmax_scale=case.scale,
                                q_rope_base=args.q_rope_base or None)
    ws = torch.empty(mla.prefill_workspace_bytes(params), dtype=torch.uint8, device="cuda")
    out = torch.empty((case.B, case.T, case.H, case.dv), dtype=torch.bfloat16, device="cuda")

    def step():
        mla.prefill_naive(q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens, out=out, workspace=ws,
                          params=params)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms = timed_back_to_back(step, args.steps)
    L = case.seqlens.astype(np.int64)
    rows = int(L.sum())
    # causal (query, key) pairs: query t at position L - T + t sees keys 0..pos
    pairs = int(sum(int(l) * case.T - case.T * (case.T - 1) // 2 for l in L))
    f_decomp = 2 * rows * case.H * case.dc * (case.dn + case.dv)
    f_attn = 2 * pairs * case.H * (case.dn + case.dr + case.dv)
    flops = f_decomp + f_attn
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "mode": "prefill", "metric": "naive causal prefill bf16 MFMA TFLOP/s (% of dense peak)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded normals; c = W_DKV x from x of width 7168)",
        "config": {"workload": case.name, "batch": case.B, "tokens": case.T, "heads": case.H,
                   "cached_tokens_total": rows, "q_rope_base": args.q_rope_base},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "algorithmic_flops_per_call": flops, "decompress_flops": f_decomp,
                     "attention_flops": f_attn},
        "timing": "the K calls back to back between one event pair"}
    if not args.no_cpu_baseline:
        import oracle
        line["cpu_baseline"] = cpu_baseline_sampled(
            lambda rr: oracle.prefill_naive(case.q_nope, case.q_rope, case.w_uk, case.w_uv,
                                            case.cache[:, :, :case.dc], case.cache[:, :, case.dc:],
                                            case.seqlens, case.scale, rr),
            [(b, t) for b in range(case.B) for t in range(case.T)], args.cpu_seconds,
            lambda t_call: flops / t_call / 1e12, "TFLOP/s", "query rows (all heads)")
    print(json.dumps(line), flush=True)
    return 0


def bench_chunk(args, mla, datagen):
    """Absorbed causal prefill (a chunk of new queries attending to a long cached
    context in latent space) on the V3 shape: batch 4, 64 queries each over
    32768 cached rows; one JSON line with the whole call's bf16 MFMA
    throughput against the dense peak."""
    import numpy as np
    import torch

    from mla_latent_kv_12_amd.tensors import to_device

    case = datagen.make_workload("v3-chunk-32k")
    dt = case.dtype
    cache = to_device(case.cache, dt)
    q_nope, q_rope = to_device(case.q_nope, dt), to_device(case.q_rope, dt)
    w_uk, w_uv = to_device(case.w_uk, dt), to_device(case.w_uv, dt)
    ckv, kpe = cache[:, :, : case.dc], cache[:, :, case.dc:]
    seqlens = torch.from_numpy(case.seqlens.astype(np.int32)).cuda()
    params = mla.prefill_params(q_nope, q_rope, w_uk, w_uv, ckv, kpe, softmax_scale=case.scale,
                                num_splits=args.splits,
                                q_rope_base=args.q_rope_base or None)
    ws = torch.empty(mla.prefill_absorbed_workspace_bytes(params), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((case.B, case.T, case.H, case.dv), dtype=torch.bfloat16, device="cuda")

    def step():
        mla.prefill_absorbed(q_nope, q_rope, w_uk, w_uv, ckv, kpe, seqlens, out=out, workspace=ws,
                             params=params)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms = timed_back_to_back(step, args.steps)
    L = case.seqlens.astype(np.int64)
    rows = case.B * case.T
    pairs = int(sum(int(l) * case.T - case.T * (case.T - 1) // 2 for l in L))
    f_absorb = 2 * rows * case.H * case.dn * case.dc
    f_attn = 2 * pairs * case.H * (2 * case.dc + case.dr)
    f_up = 2 * rows * case.H * case.dv * case.dc
    flops = f_absorb + f_attn + f_up
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "mode": "chunk", "metric": "absorbed causal prefill bf16 MFMA TFLOP/s (% of dense peak)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded normals)",
        "config": {"workload": case.name, "batch": case.B, "tokens": case.T, "heads": case.H,
                   "cached_tokens_total": int(L.sum()),
                   "splits": mla.prefill_absorbed_num_splits(params),
                   "q_rope_base": args.q_rope_base},
        "query_tokens_per_s": rows / (ms * 1e-3),
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "algorithmic_flops_per_call": flops, "attention_flops": f_attn,
                     "absorb_and_upproj_flops": f_absorb + f_up},
        "timing": "the K calls back to back between one event pair"}
    if not args.no_cpu_baseline:
        import oracle
        line["cpu_baseline"] = cpu_baseline_sampled(
            lambda rr: oracle.prefill_absorbed(case.q_nope, case.q_rope, case.w_uk, case.w_uv,
                                               case.cache[:, :, :case.dc],
                                               case.cache[:, :, case.dc:], case.seqlens,
                                               case.scale, rr),
            [(b, t) for b in range(case.B) for t in range(case.T)], args.cpu_seconds,
            lambda t_call: flops / t_call / 1e12, "TFLOP/s", "query rows (all heads)")
    print(json.dumps(line), flush=True)
    return 0


def bench_outproj(args, mla, datagen):
    """The step after decode, the output projection for batch 8 at the V3
    shape: y = W_O concat_h(out_h) (W_O 7168 x 16384, the unfolded form) and,
    for comparison, y = W_OV concat_h(o_lat_h) with W_UV folded in (W_OV 7168 x
    65536); one JSON line with both kernels' algorithmic HBM rates."""
    import numpy as np
    import torch

    B, H, dv, dc, d_model = 8, 128, 128, 512, 7168
    g = torch.Generator(device="cuda").manual_seed(20260007)

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)

    x_unf = randn(B, H * dv)
    x_fold = randn(B, H * dc)
    w_o = randn(d_model, H * dv, std=1.0 / np.sqrt(H * dv))
    w_uv = randn(H, dv, dc, std=1.0 / np.sqrt(dc))
    w_ov = mla.fold_value_output(w_o, w_uv)   # first call: also loads the kernel
    fold = []
    for _ in range(3):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        mla.fold_value_output(w_o, w_uv, out=w_ov)
        t1.record()
        torch.cuda.synchronize()
        fold.append(t0.elapsed_time(t1))
    fold_ms = float(np.median(fold))
    res = {}
    for name, x, w in (("unfolded", x_unf, w_o), ("folded", x_fold, w_ov)):
        params = mla.proj_params(x, w)
        ws = torch.empty(mla.output_proj_workspace_bytes(params), dtype=torch.uint8,
                         device="cuda")
        y = torch.empty((B, d_model), dtype=torch.bfloat16, device="cuda")

        def step():
            mla.output_proj(x, w, out=y, workspace=ws, params=params)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ref = y.clone()
        # eager calls back to back: the host's launch path (argument checks
        # and marshalling, 40-65 us) is slower than the kernel, so this
        # measures the host
        us_eager = 1e3 * timed_back_to_back(step, args.steps)
        # device time: the steps captured back to back in one HIP graph,
        # median of 3 replays, each checked against the eager result
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step()
        reps = []
        for _ in range(3):
            y.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            if not torch.equal(y, ref):
                raise RuntimeError("graph replay of the projection differs from the eager call")
            reps.append(1e3 * e0.elapsed_time(e1) / args.steps)
        us = float(np.median(reps))
        nbytes = (w.numel() + x.numel() + y.numel()) * 2
        res[name] = {"us_per_call": us, "us_per_call_eager": us_eager,
                     "weight_bytes": w.numel() * 2, "gbps": nbytes / (us * 1e-6) / 1e9,
                     "form": "direct" if ws.numel() == 0 else "sliced"}
    gbps = res["unfolded"]["gbps"]
    line = {
        "mode": "outproj", "metric": "output projection after decode, HBM GB/s (% of peak)",
        "value": gbps, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic (seeded normals)",
        "config": {"workload": "V3 output projection batch 8, d_model 7168", "batch": B,
                   "heads": H, "d_v": dv, "d_c": dc, "d_model": d_model},
        "timing": "HIP graph of the steps, median of 3 replays (eager: the host's launch rate)",
        "unfolded": res["unfolded"], "folded": res["folded"], "fold_weights_ms": fold_ms,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS,
                     "kernel": "rowproj_direct_bf16_kernel (unfolded W_O)"}}
    if not args.no_cpu_baseline:
        import oracle

        def bits(t):  # bf16 storage bits on the host, as the oracle takes them
            return t.cpu().view(torch.int16).numpy().view(np.uint16)

        xh, wh = bits(x_unf), bits(w_o)
        nbytes = (w_o.numel() + x_unf.numel() + B * d_model) * 2
        line["cpu_baseline"] = cpu_baseline_sampled(
            lambda rr: oracle.output_proj(xh[rr], wh), list(range(B)), args.cpu_seconds,
            lambda t_call: nbytes / t_call / 1e9, "GB/s", "rows of the unfolded projection")
    print(json.dumps(line), flush=True)
    return 0


def bench_append(args, mla, datagen):
    """The cache-row producer for one decode step: c = W_DKV h and the rotated
    k^R = RoPE(W_KR h) for 8 sequences (d_model 7168), written into a 128k-row
    cache; one JSON line with the algorithmic HBM rate against 8 TB/s."""
    import numpy as np
    import torch

    from mla_latent_kv_12_amd.tensors import to_device

    case = datagen.make_workload("v3-append")
    dt = case.dtype
    h, w_dkv, w_kr = to_device(case.h, dt), to_device(case.w_dkv, dt), to_device(case.w_kr, dt)
    n_max = 131072
    cache = torch.zeros((case.B, n_max, case.dc + case.dr), dtype=torch.bfloat16, device="cuda")
    pos = torch.tensor([(131071 - 977 * b) % n_max for b in range(case.B)], dtype=torch.int32,
                       device="cuda")

    def step():
        mla.cache_append(h, w_dkv, w_kr, pos, cache[:, :, :case.dc], cache[:, :, case.dc:])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rows, cols = torch.arange(case.B, device="cuda"), pos.long()
    ref = cache[rows, cols].clone()
    # eager calls, one event pair each: for a kernel this small the host's
    # launch rate, not the device, sets this figure
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    us_eager = 1e3 * float(np.mean(per))
    # device time: the steps captured back to back in one HIP graph; each
    # replay is checked against the eager result (its rows cleared first)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()
    reps = []
    for _ in range(3):
        cache[rows, cols] = 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        if not torch.equal(cache[rows, cols], ref):
            raise RuntimeError("graph replay of the append differs from the eager call")
        reps.append(1e3 * e0.elapsed_time(e1) / args.steps)
    us = float(np.median(reps))
    nbytes = ((case.dc + case.dr) * case.d_model + case.B * case.d_model
              + case.B * (case.dc + case.dr)) * 2
    gbps = nbytes / (us * 1e-6) / 1e9
    line = {
        "mode": "append", "metric": "cache-row producer HBM GB/s (% of peak)", "value": gbps,
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "us_per_step": us, "us_per_call_eager": us_eager,
        "timing": "HIP graph of the steps, median of 3 replays", "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded normals)",
        "config": {"workload": case.name, "batch": case.B, "d_model": case.d_model,
                   "d_c": case.dc, "d_r": case.dr},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "algorithmic_bytes_per_call": nbytes},
        "eager_us_p10_p90": [1e3 * float(np.percentile(per, 10)),
                             1e3 * float(np.percentile(per, 90))]}
    if not args.no_cpu_baseline:
        import oracle
        pos_h = pos.cpu().numpy()
        line["cpu_baseline"] = cpu_baseline_sampled(
            lambda rr: oracle.cache_rows(case.h[rr], case.w_dkv, case.w_kr, pos_h[rr]),
            list(range(case.B)), args.cpu_seconds, lambda t_call: nbytes / t_call / 1e9, "GB/s",
            "sequences")
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3-128k", choices=["v3-4k", "v3-ragged", "v3-128k"],
                    help="decode workload (v3-128k: V3 shape, batch 8, 131072 cached tokens)")
    ap.add_argument("--splits", type=int, default=0, help="context splits (0 = library's choice)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--q-rope-base", type=float, default=0.0,
                    help="rotate q_rope in the library at each query's position with this base "
                         "(0: q_rope is taken as already rotated)")
    ap.add_argument("--mode", choices=["decode", "prefill", "chunk", "append", "outproj", "copy"],
                    default="decode",
                    help="prefill: the naive causal prefill (V3 shape, T=4096) against the bf16 "
                         "MFMA peak; chunk: the absorbed prefill of 64 queries per sequence over "
                         "32768 cached rows (batch 4); append: the cache-row producer (batch 8, "
                         "d_model 7168); outproj: the output projection after decode, unfolded "
                         "and with W_UV folded in "
                         "against HBM; copy: a plain device-to-device copy of --copy-bytes, the "
                         "reference that scales the profiler's byte counters")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--rotate", type=int, default=1,
                    help="distinct input copies cycled through (>1 defeats the 256 MB MALL "
                         "for the small workloads)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path across "
                                   "several GPUs (context or batch sharding) is a design only",
                          "n_gpus": args.gpus}), flush=True)
        return 2

    import numpy as np
    import torch

    if args.mode == "copy":
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        print(json.dumps({"mode": "copy", "bytes_read": args.copy_bytes,
                          "bytes_written": args.copy_bytes, "ms_per_copy": ms,
                          "gbps": 2 * args.copy_bytes / (ms * 1e-3) / 1e9}), flush=True)
        return 0

    import mla_latent_kv_12_amd as mla
    from mla_latent_kv_12_amd import datagen
    from mla_latent_kv_12_amd.tensors import decode_tensors

    if args.mode == "prefill":
        return bench_prefill(args, mla, datagen)
    if args.mode == "chunk":
        return bench_chunk(args, mla, datagen)
    if args.mode == "append":
        return bench_append(args, mla, datagen)
    if args.mode == "outproj":
        return bench_outproj(args, mla, datagen)

    t_gen = time.perf_counter()
    case = datagen.make_workload(args.workload)
    print(f"# generated {case.name} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)
    copies = [decode_tensors(case) for _ in range(max(1, args.rotate))]
    t = copies[0]
    params = mla.decode_params(t["q_nope"], t["q_rope"], t["w_uk"], t["w_uv"], t["ckv_cache"],
                               t["kpe_cache"], softmax_scale=case.scale, num_splits=args.splits,
                               q_rope_base=args.q_rope_base or None)
    splits = mla.decode_num_splits(params)
    ws = torch.empty(mla.decode_workspace_bytes(params), dtype=torch.uint8, device="cuda")
    out = torch.empty((case.B, case.H, case.dv), dtype=torch.bfloat16, device="cuda")

    def step(i, events=None):
        c = copies[i % len(copies)]
        mla.decode(c["q_nope"], c["q_rope"], c["w_uk"], c["w_uv"], c["ckv_cache"],
                   c["kpe_cache"], c["seqlens"], out=out, workspace=ws, params=params,
                   events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    # Pass 1 (value): the K calls back to back between one event pair, with
    # nothing recorded between them.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(K):
        step(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    # Pass 2 (roofline): K more calls, each with two fence-free HIP events
    # recorded on the launch stream around its split-KV kernel (each record
    # idles the GPU for a few microseconds, which is why pass 1 has none).
    ev = HipEvents(2 * K)
    torch.cuda.synchronize()
    for i in range(K):
        step(i, events=ev.around_attention(2 * i))
    torch.cuda.synchronize()
    attn = [ev.ms(2 * i, 2 * i + 1) for i in range(K)]
    ev.close()

    # Pass 3 (context, not `value`): the same K event-free calls once the
    # chip's clock has settled.  Under this load the clock controller lets
    # the first calls of a run through at a high clock, then throttles hard
    # and settles in between within about 100 calls, so a short run times
    # the transient; this pass times K calls after STEADY_SETTLE more.
    for i in range(STEADY_SETTLE):
        step(i)
    s3, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s3.record()
    for i in range(K):
        step(i)
    e3.record()
    torch.cuda.synchronize()
    steady_ms = s3.elapsed_time(e3) / K

    ms_per_step = total_ms / K
    seq = case.seqlens.astype(np.int64)
    rows = int(seq.sum())
    row_bytes = (case.dc + case.dr) * 2
    cache_bytes = rows * row_bytes
    weight_bytes = 2 * case.H * case.dn * case.dc * 2
    qo_bytes = case.B * case.H * (case.dn + case.dr + case.dv) * 2
    call_bytes = cache_bytes + weight_bytes + qo_bytes
    flops = 2 * rows * case.H * (case.dc + case.dr + case.dc) + 4 * case.B * case.H * case.dn * case.dc
    attn_ms = float(np.mean(attn))
    attn_gbps = cache_bytes / (attn_ms * 1e-3) / 1e9
    call_gbps = call_bytes / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": case.B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normals; random-init weights of the V3 shape)",
        "config": {"workload": case.name, "batch": case.B, "heads": case.H, "d_c": case.dc,
                   "d_r": case.dr, "d_n": case.dn, "d_v": case.dv,
                   "cached_tokens_total": rows, "splits": splits, "input_copies": len(copies),
                   "q_rope_base": args.q_rope_base},
        "hbm_gbps_call": call_gbps,
        "hbm_frac_call": call_gbps / HBM_PEAK_GBPS,
        "context_rows_per_s": rows / (ms_per_step * 1e-3),
        "mfma_tflops_call": flops / (ms_per_step * 1e-3) / 1e12,
        "wall_s_timed": wall,
        "timing": ("value: the K calls back to back between one event pair (no other events); "
                   "stages_us and roofline: a second pass of K calls with hipEvents without the "
                   "system fence around each call's split-KV kernel"),
        "steady_state": {"ms_per_step": steady_ms, "tokens_per_s": case.B / (steady_ms * 1e-3),
                         "settle_calls": STEADY_SETTLE,
                         "note": "context only: K more event-free calls after the settle calls"},
        "stages_us": {"splitkv_attention": 1e3 * attn_ms,
                      "splitkv_p10_p90": [1e3 * float(np.percentile(attn, 10)),
                                          1e3 * float(np.percentile(attn, 90))]},
        "roofline": {"bound": "hbm", "achieved": attn_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": attn_gbps / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(args.workload == "v3-128k" and args.splits in (0, 32)
                                                 and not args.q_rope_base),
                     "kernel": "decode_splitkv_bf16_kernel",
                     "algorithmic_bytes_per_launch": cache_bytes},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
