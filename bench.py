#!/usr/bin/env python3
"""Benchmark of one decode step over a vector-quantized KV cache on one MI355X.

A step is one pass of the whole hot path for one layer: append the new token's
key and value as codes (smoothing + Hadamard + nearest centroid), transform the
query, split-context attention over the codes, and the log-sum-exp combine.
Inputs are synthetic and resident in HBM before the timed region; codebooks
are trained on the GPU (20 Lloyd iterations on a 4096-token calibration draw).

Prints one JSON line.  `value` is algorithmic HBM bytes of the step divided by
the measured step time (GB/s).  The headline workload is the Llama-3.1-8B
attention shape at batch 32 and 196,608 tokens with a 2-bit cache; the
batch-1 shape at the same context is reported alongside.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "2-bit VQ decode-attn us/step + HBM GB/s (% peak), 8B shape @196k; x vs bf16"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20

_head = {}
RUNS = 5                      # timed runs per figure: the median is reported, with p10 and p90


def pct(xs, p):
    """Nearest-rank p-quantile of xs (p in [0, 1])."""
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(p * (len(xs) - 1)))))]


def host_cpu():
    """The host CPU's model name and the number of CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))

# HBM traffic of the decode kernel comes from rocprofv3 counters recorded in
# this file, valid only while the kernel sources still hash to the recorded value.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_mfma_kernel__llama8b_b32_t196k__hbm_traffic.txt")
KERNEL_SOURCES = ["decode.hip", "attn_common.h", "device_util.h", "internal.h", "qtransform.h", "token_search.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "vector_quantized_bit_vqkv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per decode launch from the committed counter summary, or None."""
    if workload != "llama8b_b32_t196k" or not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    return int(fields["hbm_bytes_per_launch"])


def head_start(dev, ms=12.0):
    """Enqueue about `ms` of HBM read-stream work so that the host can queue every
    timed launch before the GPU reaches them: the timed steps then run back to
    back and the events bracket GPU time only, not Python launch overhead."""
    import torch
    import vector_quantized_bit_vqkv_amd as vq
    if "buf" not in _head:
        _head["buf"] = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        _head["sink"] = torch.zeros(1024, dtype=torch.int32, device=dev)
    for _ in range(max(1, int(ms / 0.2))):      # ~0.2 ms per 1 GB read
        vq.baseline_read_stream(_head["buf"], _head["sink"], 8192)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b_b32_t196k")
    ap.add_argument("--also", default="llama8b_b1_t196k,llama8b_b1_t32k,qwen14b_b8_t128k_1p5,llama8b_b8_t196k_3bit,"
                                      "qwen14b_b8_t128k_1p25,llama8b_b8_t196k_4bit",
                    help="comma-separated extra workloads reported under 'also' ('' for none)")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bf16 baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    ap.add_argument("--decode-path", default="", choices=["", "table", "gather", "mfma"],
                    help="time the decode on another kernel (measurement; the four separate calls)")
    return ap.parse_args()


class Workload:
    """Device-resident state of one workload: calibration, codebooks, codes, step inputs."""

    def __init__(self, name, dev, keep_bf16, keep_inputs=False):
        import torch

        import synth
        import vector_quantized_bit_vqkv_amd as vq
        self.name = name
        wl = synth.WORKLOADS[name]
        self.wl = wl
        B, Hq, Hkv, T, fmt = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.seq_len, wl.fmt
        E, dsub, J = wl.entries, wl.dsub, wl.nsub
        seed = synth.seed_for(name)
        t0 = time.time()
        case = synth.make_device_case(wl, seed, dev)
        torch.cuda.synchronize()
        self.gen_s = time.time() - t0

        # Offline calibration on the GPU: smoothing scales, K-Means codebooks.
        t0 = time.time()
        self.smooth = torch.empty((Hkv, 128), dtype=torch.float32, device=dev)
        vq.smooth_scales(case["k_cal"], self.smooth)
        self.k_book = torch.empty((Hkv, E, dsub), dtype=torch.int16, device=dev)
        self.v_book = torch.empty((Hkv, E, dsub), dtype=torch.int16, device=dev)
        n_cal = case["k_cal"].shape[1]
        ws = torch.empty(vq.train_workspace_bytes(fmt, n_cal), dtype=torch.uint8, device=dev)
        for h in range(Hkv):
            ik = torch.from_numpy(synth.kmeans_init_indices(seed + 2 * h, n_cal * J, E)).to(dev)
            iv = torch.from_numpy(synth.kmeans_init_indices(seed + 2 * h + 1, n_cal * J, E)).to(dev)
            vq.train_codebook(fmt, case["k_cal"][h], True, self.smooth[h], ik, 20, self.k_book[h], ws)
            vq.train_codebook(fmt, case["v_cal"][h], False, None, iv, 20, self.v_book[h], ws)
        torch.cuda.synchronize()
        self.calib_s = time.time() - t0
        del ws

        # The context: T tokens, the last of which is the step's new token.
        self.shape = vq.make_shape(B, Hq, Hkv, T, fmt)
        W = vq.code_bytes_per_token(fmt)
        k_codes = torch.empty((B, Hkv, T * W), dtype=torch.uint8, device=dev)
        v_codes = torch.empty((B, Hkv, T * W), dtype=torch.uint8, device=dev)
        t0 = time.time()
        vq.quantize_append(self.shape, case["k"], case["v"], 0, self.smooth, self.k_book, self.v_book,
                           k_codes, v_codes)
        torch.cuda.synchronize()
        self.prefill_s = time.time() - t0
        self.k_new = case["k"][:, :, T - 1:T].contiguous()
        self.v_new = case["v"][:, :, T - 1:T].contiguous()
        self.q = case["q"]
        # Rotate over R copies so the step's working set exceeds the 256 MB
        # last-level cache: every step then reads its codes from HBM.
        self.code_bytes = 2 * B * Hkv * T * W
        R = max(1, math.ceil(2 * MALL_BYTES / self.code_bytes))
        self.caches = [(k_codes, v_codes)] + [(k_codes.clone(), v_codes.clone()) for _ in range(R - 1)]
        self.k_bf16 = case["k"] if keep_bf16 else None
        self.v_bf16 = case["v"] if keep_bf16 else None
        # The drawn inputs (calibration rows, keys, values, queries), kept for
        # checking against the oracle; the benchmark itself drops them.
        self.case = case if keep_inputs else None
        self.seed = seed
        del case
        self.decode_path = ""
        self.S = vq.suggest_splits(self.shape, T)
        self.q_prime = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        self.workspace = torch.empty(vq.workspace_bytes(self.shape, self.S), dtype=torch.uint8, device=dev)
        self.step_workspace = torch.empty(vq.step_workspace_bytes(self.shape, self.S), dtype=torch.uint8, device=dev)

        # Algorithmic bytes (what the method must move), per launch / per step.
        book_bytes = 2 * Hkv * E * dsub * 2
        self.decode_bytes = self.code_bytes + book_bytes + B * Hq * 128 * 4            # codes, books, q'
        self.step_bytes = (self.code_bytes + book_bytes                                  # attention reads
                           + B * Hq * 128 * 2 + Hkv * 128 * 4                           # q (bf16), s
                           + B * Hq * 128 * 4                                           # out (fp32)
                           + 2 * B * Hkv * 128 * 2 + 2 * B * Hkv * W)                   # new k, v; new codes

    def decode(self, kc, vc):
        """The attention pass as vqkv_decode_attention launches it (or, for
        measurement, on the kernel named by decode_path)."""
        import vector_quantized_bit_vqkv_amd as vq
        T = self.wl.seq_len
        if self.decode_path:
            vq.measure_decode_attention(self.shape, self.q_prime, self.k_book, self.v_book, kc, vc, T, self.S,
                                        self.workspace, self.decode_path)
        else:
            vq.decode_attention(self.shape, self.q_prime, self.k_book, self.v_book, kc, vc, T, self.S,
                                self.workspace)

    def step(self, i):
        import vector_quantized_bit_vqkv_amd as vq
        kc, vc = self.caches[i % len(self.caches)]
        T = self.wl.seq_len
        vq.quantize_append(self.shape, self.k_new, self.v_new, T - 1, self.smooth, self.k_book, self.v_book, kc, vc)
        vq.transform_query(self.shape, self.q, self.smooth, self.q_prime)
        self.decode(kc, vc)
        vq.combine(self.shape, self.S, self.workspace, self.out)

    def fused_step(self, i):
        import vector_quantized_bit_vqkv_amd as vq
        kc, vc = self.caches[i % len(self.caches)]
        T = self.wl.seq_len
        vq.decode_step(self.shape, self.q, self.k_new, self.v_new, T - 1, self.smooth, self.k_book, self.v_book,
                       kc, vc, self.S, self.step_workspace, self.out)

    def time_fused_steps(self, steps, warmup, runs=RUNS):
        """The same step through decode_step: the combine fused into the decode, and with one
        2-bit split the append too (one launch; else the append is a launch of its own).
        Returns the mean ms per step of each of `runs` timed runs of exactly `steps` steps."""
        return self._time_runs(self.fused_step, steps, warmup, runs)

    def _time_runs(self, fn, steps, warmup, runs):
        """Mean ms per call of `steps` back-to-back calls fn(i), for each of `runs`
        runs, bracketed by HIP events on torch's current stream (the stream every
        call launches on)."""
        import torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        per_run = []
        for r in range(runs):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            head_start(self.q.device)
            start.record()
            for i in range(steps):
                fn(warmup + r * steps + i)
            end.record()
            torch.cuda.synchronize()
            per_run.append(start.elapsed_time(end) / steps)
        return per_run

    def time_steps(self, steps, warmup, runs=RUNS):
        """The step as four separate calls: mean ms per step of each run."""
        return self._time_runs(self.step, steps, warmup, runs)

    def time_decode(self, steps, warmup, runs=RUNS):
        """The attention pass alone (vqkv_decode_attention), back to back over the
        rotated cache copies: mean ms per launch of each run.  (Events around
        single launches in a mixed stream add their own recording to each
        launch, several us at batch 1; back-to-back launches do not.)"""
        import vector_quantized_bit_vqkv_amd as vq
        vq.transform_query(self.shape, self.q, self.smooth, self.q_prime)

        def once(i):
            kc, vc = self.caches[i % len(self.caches)]
            self.decode(kc, vc)
        return self._time_runs(once, steps, warmup, runs)

    def time_parts(self, steps, warmup):
        """The step's two small calls on their own, back to back: the one-token
        append (vqkv_quantize_append, all sequences and KV heads) and the query
        transform; median ms per call of each."""
        import vector_quantized_bit_vqkv_amd as vq
        T = self.wl.seq_len

        def append(i):
            kc, vc = self.caches[i % len(self.caches)]
            vq.quantize_append(self.shape, self.k_new, self.v_new, T - 1, self.smooth, self.k_book, self.v_book,
                               kc, vc)

        def transform(i):
            vq.transform_query(self.shape, self.q, self.smooth, self.q_prime)
        return (pct(self._time_runs(append, steps, warmup, RUNS), 0.5),
                pct(self._time_runs(transform, steps, warmup, RUNS), 0.5))

    def time_attention_only(self, steps, warmup):
        """decode + combine only (what the bf16 comparison times)."""
        import torch
        import vector_quantized_bit_vqkv_amd as vq
        T = self.wl.seq_len

        def once(i):
            kc, vc = self.caches[i % len(self.caches)]
            self.decode(kc, vc)
            vq.combine(self.shape, self.S, self.workspace, self.out)
        return pct(self._time_runs(once, steps, warmup, RUNS), 0.5)

    def time_bf16(self, steps, warmup):
        """The same attention over the unquantized bf16 cache (bf16 decode + combine),
        at the best of a few split counts (the bf16 kernel keeps more work-groups
        per CU than the VQ kernel, so it wants more splits)."""
        import torch
        import vector_quantized_bit_vqkv_amd as vq
        T = self.wl.seq_len
        best = None
        for S in sorted({self.S, 2 * self.S, 4 * self.S}):
            if S > (T + 63) // 64:
                continue
            ws = torch.empty(vq.workspace_bytes(self.shape, S), dtype=torch.uint8, device=self.q.device)

            def once():
                vq.baseline_bf16_decode(self.shape, self.q, self.k_bf16, self.v_bf16, T, S, ws)
                vq.combine(self.shape, S, ws, self.out)
            for _ in range(warmup):
                once()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            head_start(self.q.device)
            a.record()
            for _ in range(steps):
                once()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / steps
            if best is None or ms < best[0]:
                best = (ms, S)
            del ws
        ms, S = best
        wl = self.wl
        bf16_bytes = 2 * wl.batch * wl.num_kv_heads * T * 128 * 2
        return ms, bf16_bytes / (ms * 1e-3) / 1e9, S

    def cpu_baseline(self, budget_s):
        """The CPU oracle on a bounded sample of this step: whole sequences (all
        query heads, full context), attention plus the append's quantization,
        timed until the budget is spent, then scaled to the full batch; first on
        every CPU this process may use, then on one thread (a quarter of the
        budget, at least one sequence)."""
        import numpy as np

        import oracle
        wl = self.wl
        B, Hq, Hkv, T, fmt = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.seq_len, wl.fmt
        threads = oracle.default_threads()
        model, affinity = host_cpu()
        kb = self.k_book.cpu().numpy().view(np.uint16)
        vb = self.v_book.cpu().numpy().view(np.uint16)
        s = self.smooth.cpu().numpy()
        q = self.q.float().cpu().numpy()
        kn = self.k_new.float().cpu().numpy()
        vn = self.v_new.float().cpu().numpy()
        kc_dev, vc_dev = self.caches[0]
        kept = []

        def sequence(i):
            # Sequences in order, each unpacked once (outside the timing); past
            # the batch, the first few are timed again.
            if i < B:
                kc = np.stack([oracle.unpack_k(fmt, kc_dev[i, h].cpu().numpy(), T) for h in range(Hkv)])[None]
                vc = np.stack([oracle.unpack_v(fmt, vc_dev[i, h].cpu().numpy(), T) for h in range(Hkv)])[None]
                if len(kept) < 4:
                    kept.append((i, kc, vc))
                return i, kc, vc
            return kept[(i - B) % len(kept)]

        def timed(nthreads, budget):
            spent, done = 0.0, 0
            while spent < budget or done == 0:
                b, kc, vc = sequence(done)
                t0 = time.perf_counter()
                for h in range(Hkv):
                    oracle.quantize(fmt, kn[b, h], vn[b, h], s[h], kb[h], vb[h], nthreads=nthreads)
                oracle.attention(fmt, q[b:b + 1], s, kb, vb, kc, vc, nthreads=nthreads)
                spent += time.perf_counter() - t0
                done += 1
            return spent, done

        spent, done = timed(threads, budget_s)
        full_s = spent / done * B
        spent1, done1 = timed(1, budget_s / 4)
        full1 = spent1 / done1 * B
        what = (f"sequence computations (all {Hq} q-heads, {T} tokens each: fp64 oracle attention plus "
                f"quantization of the appended token), scaled to the batch of {B}")
        return {"value": round(self.step_bytes / full_s / 1e9, 3), "unit": "GB/s", "cores": threads,
                "kind": "oracle",
                "sample": f"{done} {what}, {spent:.1f} s on {threads} threads",
                "us_per_step": round(full_s * 1e6, 1),
                "cpu_model": model, "cpus_available": affinity,
                "one_thread": {"value": round(self.step_bytes / full1 / 1e9, 4), "unit": "GB/s",
                               "us_per_step": round(full1 * 1e6, 1),
                               "sample": f"{done1} {what}, {spent1:.1f} s on 1 thread"}}


def read_stream_peak(dev):
    import torch
    import vector_quantized_bit_vqkv_amd as vq
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    for _ in range(3):
        vq.baseline_read_stream(buf, sink, 2048)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    n = 10
    for _ in range(n):
        vq.baseline_read_stream(buf, sink, 2048)
    b.record()
    torch.cuda.synchronize()
    gbps = buf.numel() * n / (a.elapsed_time(b) * 1e-3) / 1e9
    del buf
    return gbps


def measure(name, args, dev, with_bf16, with_cpu):
    import torch
    wk = Workload(name, dev, keep_bf16=with_bf16)
    wk.decode_path = args.decode_path
    four_runs = wk.time_steps(args.steps, args.warmup)
    # The product step is decode_step; a measurement override of the decode
    # kernel applies to the four separate calls only, so it times those.
    step_runs = four_runs if args.decode_path else wk.time_fused_steps(args.steps, args.warmup)
    step_ms, four_ms = pct(step_runs, 0.5), pct(four_runs, 0.5)
    dec = wk.time_decode(args.steps, args.warmup)
    dec_ms = sum(dec) / len(dec)                  # every run has the same number of launches
    attn_ms = wk.time_attention_only(args.steps, args.warmup)
    append_ms, transform_ms = wk.time_parts(args.steps, args.warmup)
    res = {
        "workload": name,
        "us_per_step": round(step_ms * 1e3, 2),
        "us_per_step_p10": round(pct(step_runs, 0.1) * 1e3, 2),
        "us_per_step_p90": round(pct(step_runs, 0.9) * 1e3, 2),
        "us_per_step_runs": [round(x * 1e3, 2) for x in step_runs],
        "us_per_step_four_calls": round(four_ms * 1e3, 2),
        "step_call": "four calls" if args.decode_path else "decode_step",
        "GBps": round(wk.step_bytes / (step_ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100 * wk.step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
        "decode_us": round(dec_ms * 1e3, 2),
        "decode_us_median": round(pct(dec, 0.5) * 1e3, 2),
        "decode_us_p10": round(pct(dec, 0.1) * 1e3, 2),
        "decode_us_p90": round(pct(dec, 0.9) * 1e3, 2),
        "decode_launches": len(dec) * args.steps,
        "decode_GBps": round(wk.decode_bytes / (dec_ms * 1e-3) / 1e9, 1),
        "attention_us": round(attn_ms * 1e3, 2),
        "append_us": round(append_ms * 1e3, 2),
        "transform_query_us": round(transform_ms * 1e3, 2),
        "num_splits": wk.S,
        "cache_copies": len(wk.caches),
        "step_bytes": wk.step_bytes,
        "decode_bytes": wk.decode_bytes,
        "setup_s": {"generate": round(wk.gen_s, 2), "calibrate": round(wk.calib_s, 2),
                    "prefill_quantize": round(wk.prefill_s, 2)},
        # Bulk append of the whole context (one call, wall clock, first launch included).
        "prefill_Mtoken_heads_per_s": round(wk.wl.batch * wk.wl.num_kv_heads * wk.wl.seq_len / wk.prefill_s / 1e6, 1),
    }
    if with_bf16:
        bf_ms, bf_gbps, bf_S = wk.time_bf16(max(5, args.steps // 5), 2)
        res["bf16_attention_us"] = round(bf_ms * 1e3, 2)
        res["bf16_GBps"] = round(bf_gbps, 1)
        res["bf16_num_splits"] = bf_S
        res["speedup_vs_bf16"] = round(bf_ms / attn_ms, 2)
        res["speedup_vs_bf16_step"] = round(bf_ms / step_ms, 2)
    cpu = wk.cpu_baseline(args.cpu_seconds) if with_cpu else None
    del wk
    torch.cuda.empty_cache()
    return res, cpu


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): this path "
              "has no multi-GPU mode; shard by KV head or context across GPUs as described in the design notes.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    import vector_quantized_bit_vqkv_amd as vq
    vq.lib()

    head, cpu = measure(args.workload, args, dev, not args.no_bf16, not args.no_cpu_baseline)
    also = []
    for name in [n for n in args.also.split(",") if n and n != args.workload]:
        r, _ = measure(name, args, dev, not args.no_bf16, False)
        also.append(r)
    stream_gbps = read_stream_peak(dev)

    achieved = head["decode_GBps"]
    for r in [head] + also:                      # against this box's own read stream
        r["decode_pct_read_stream"] = round(100 * r["decode_GBps"] / stream_gbps, 1)
    line = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": 32, "q_heads": 32, "kv_heads": 8, "seq_len": 196608,
                   "format": "2-bit, 256x4 fp16 codebooks, uint8 codes",
                   "arithmetic": "fp16 products with fp32 accumulation (MFMA); fp32 softmax"}
        if args.workload == "llama8b_b32_t196k"
        else {"workload": args.workload},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(args.workload),
                     "kernel": "decode_mfma_kernel", "per_launch_bytes": head["decode_bytes"],
                     "avg_launch_us": head["decode_us"]},
        "cpu_baseline": cpu,
        "detail": head,
        "also": also,
        "read_stream_GBps": round(stream_gbps, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
