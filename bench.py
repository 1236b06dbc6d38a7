#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one pass of the path over one batch of synthetic input: the state
buffer is initialised (zero fill) and the chunked prefill runs over a Ling-shaped
KDA layer (B=1, H=64, T=8192, d_k = d_v = 128, chunk 64, bf16 q/k/v, fp32 g,
beta and state).  ``value`` is that prefill's whole-job throughput in tokens/s,
inputs resident in HBM.  The batched decode step (B=256 sequences x 64 heads,
one token each, fp32 128x128 states) is timed in the same run and reported as
achieved state bandwidth under ``decode``.

Prints one JSON line.  ``--gpus`` above 1 is refused: the library's path runs on
one GPU (one GPU's share of the heads).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
METRIC = "KDA layer tokens/s (H=64,d=128 prefill); decode state GB/s vs HBM peak"
# Context from the pages, not targets.  Page "Ling-3.1-flash and the 7:1 hybrid: how
# much KV cache does a 560B model need at 1M tokens?": the model's 63 KDA layers keep a
# constant fp32 state of 264.2 MB per sequence (section "How big is the cache per token,
# exactly?"), and the Kimi Linear report claims up to 6x faster decoding at 1M tokens for
# its hybrid against full attention, on hardware the page does not name (section "Why
# would a model keep only 9 full-attention layers?").
KDA_LAYERS = 63
KIMI_LINEAR_DECODE_CLAIM = ("up to 6x faster decoding at 1M tokens (Kimi Linear hybrid "
                            "against full attention; hardware not stated)")
# The prefill is one call of kda_prefill_chunked: per window of up to 32 chunks, a
# chunk-parallel operand kernel (prep_kernel) then the state pass (state_kernel).
# Its roofline is taken over the whole call.
PREFILL_KERNEL = "prefill"
PREFILL_KERNELS = "prep_kernel + state_kernel (kda_prefill_split.hip), all windows of one call"
DECODE_KERNEL = "decode_kernel"
DECODE_TOKENS_KERNEL = "decode_kernel_4tok"  # traffic record of the 4-token decode
DECODE_BF16_KERNEL = "decode_kernel_bf16state"  # traffic record of the bf16-state decode
CONV_KERNEL = "conv_prefill"  # traffic record of the mixer front end (3 conv launches)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
_CSRC = os.path.join(ROOT, "gated_delta_rule_99_amd", "csrc")
SOURCES = {
    PREFILL_KERNEL: [os.path.join(_CSRC, "kda_prefill_split.hip"),
                     os.path.join(_CSRC, "kda_prep_tile.h"),
                     os.path.join(_CSRC, "kda_chunk_ops.h"),
                     os.path.join(_CSRC, "kda_state_pass.h")],
    DECODE_KERNEL: [os.path.join(_CSRC, "kda_decode.hip")],
    DECODE_TOKENS_KERNEL: [os.path.join(_CSRC, "kda_decode.hip")],
    DECODE_BF16_KERNEL: [os.path.join(_CSRC, "kda_decode.hip")],
    CONV_KERNEL: [os.path.join(_CSRC, "kda_conv.hip")],
}


def source_sha(kernel):
    """First 16 hex digits of sha256 over the kernel's source files, in order."""
    h = hashlib.sha256()
    for path in SOURCES[kernel]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch (for the prefill: per call, summed over its dispatches)
    from the committed rocprofv3 counter summary, scaled by the copy-kernel
    calibration; None if absent or taken on other kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return (rec["fetch_kib"] * 1024 * rec["fetch_scale"] +
            rec["write_kib"] * 1024 * rec["write_scale"])


def measured_mfma_busy(kernel):
    """Share of SIMD cycles the matrix cores were busy over the kernel's
    dispatches (SQ_VALU_MFMA_BUSY_CYCLES over SQ_BUSY_CU_CYCLES x 4 SIMDs) from
    the committed counter record; None if absent or taken on other source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    m = rec.get("mfma")
    if m is None or rec.get("source_sha") != source_sha(kernel):
        return None
    return m["mfma_busy_cycles"] / (m["sq_busy_cu_cycles"] * m["simds_per_cu"])


def prefill_algorithmic(T, H, d, chunk, with_s0, with_sfinal, g_bytes=4):
    """Algorithmic HBM bytes and flops of one prefill launch (bf16 q/k/v/o, fp32
    g/beta/state).  Bytes per token-head: q, k, v 3*2d, g 4d (2d for the bf16
    decay projection of the fused gate prologue), beta 4, o 2d.
    Flops per token-head: 6 d^2 (W S, Qt S, Kb^T U) + 5 C d (the C x C products
    and the two C-wide applications) + C^2 / 3 (triangular inverse)."""
    th = T * H
    bytes_ = th * (3 * 2 * d + g_bytes * d + 4 + 2 * d)
    state = H * d * d * 4
    bytes_ += state * (int(with_s0) + int(with_sfinal))
    flops = th * (6 * d * d + 5 * chunk * d + chunk * chunk / 3.0)
    return bytes_, flops


def decode_algorithmic(B, H, d, n_tok=1, state_bytes=4):
    """Per (sequence, head): state read + write once (2 * state_bytes * d^2) and,
    per token, q, k, v, g, beta, o."""
    return B * H * (2 * state_bytes * d * d + n_tok * (3 * 2 * d + 4 * d + 4 + 2 * d))


def cpu_baseline_run(inp):
    """The oracle's plain fp32 recurrence, as it stands, on every head of the
    prefill workload, with every host core this process may use."""
    import numpy as np
    import oracle

    cores = len(os.sched_getaffinity(0))
    q = inp.q.float().numpy()
    k = inp.k.float().numpy()
    v = inp.v.float().numpy()
    g = inp.g.numpy()
    beta = inp.beta.numpy()
    t0 = time.perf_counter()
    oracle.recurrence(q, k, v, g, beta, cu_seqlens=inp.cu_seqlens.numpy(), precision="f32",
                      n_threads=cores)
    dt = time.perf_counter() - t0
    # one thread, on a sample of the heads, scaled to the whole layer
    hs = 4
    sl = lambda x: np.ascontiguousarray(x[:, :hs])
    t0 = time.perf_counter()
    oracle.recurrence(sl(q), sl(k), sl(v), sl(g), sl(beta), cu_seqlens=inp.cu_seqlens.numpy(),
                      precision="f32", n_threads=1)
    dt1 = (time.perf_counter() - t0) * inp.H / hs
    return {"value": inp.T / dt, "unit": "tokens/s", "cores": cores, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"whole prefill workload (T={inp.T}, H={inp.H}, d={inp.d}), fp32 "
                      f"sequential recurrence, OpenMP over heads; {dt:.2f} s wall",
            "seconds": round(dt, 3),
            "single_thread": {"value": inp.T / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{hs} of the {inp.H} heads, time scaled by "
                                        f"{inp.H // hs}"}}


def cpu_decode_single_thread(inp, n_sample=32):
    """The oracle on one thread for a decode step of the batched decode workload
    (each sequence one token from its initial state), on a sample of sequences,
    scaled to the whole batch."""
    import numpy as np
    import oracle

    rows = slice(0, n_sample)
    f = lambda x: np.ascontiguousarray(x[rows].float().numpy())
    t0 = time.perf_counter()
    oracle.recurrence(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta),
                      cu_seqlens=np.arange(n_sample + 1, dtype=np.int32), S0=f(inp.S0),
                      precision="f32", n_threads=1)
    dt = (time.perf_counter() - t0) * inp.n_seqs / n_sample
    return {"value": inp.n_seqs / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_sample} of the {inp.n_seqs} sequences, time scaled by "
                      f"{inp.n_seqs // n_sample}"}


def copy_bandwidth(dev, reps=20):
    """The library's streaming copy (kda_device_copy: 16-byte non-temporal loads
    and stores, four pieces per lane in flight) of 1 GiB, read plus written bytes
    over the time: the bandwidth a streaming kernel reaches on this device."""
    import torch

    import gated_delta_rule_99_amd as kda

    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        kda.kda_device_copy(b, a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        kda.kda_device_copy(b, a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults measure steady state: on MI355X the first tens of calls of a run
    # are up to 10% slower or faster than the rest (prefill, 20 steps after 5
    # warm-ups: 0.426 ms per step; 100 after 20: 0.384; 300 after 50: 0.385).
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=500)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "prefill_gate_proj", "prefill_out_gate", "decode",
                                       "decode_tokens", "decode_bf16_state", "conv", "copy"],
                    default=None, help="run just one kernel (for profiler runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the KDA hot path runs on one GPU (one GPU's share of the heads); "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_99_amd as kda
    import workloads

    kda.load()
    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)

    if args.only == "copy":
        # the library's streaming copy of a known size: calibrates the
        # profiler's byte counters (FETCH_SIZE and WRITE_SIZE per dispatch)
        n = 1 << 28  # 1 GiB of fp32
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(max(1, args.steps)):
            kda.kda_device_copy(b, a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4}))
        return

    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic"}

    if args.only in (None, "prefill"):
        inp = workloads.ling_prefill()
        T, H, d, C = inp.T, inp.H, inp.d, inp.chunk
        q, k, v, g, beta = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
        cu = inp.cu_seqlens.to(dev)
        state = torch.empty((1, H, d, d), dtype=torch.float32, device=dev)
        o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()

        def step(e0=None, e1=None):
            kda.kda_state_init(state)
            if e0 is not None:
                e0.record()
            kda.kda_prefill_chunked(q, k, v, g, beta, cu_seqlens=cu,
                                    cu_seqlens_host=inp.cu_seqlens, chunk=C,
                                    initial_state=state, final_state=state, o=o)
            if e1 is not None:
                e1.record()

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        pairs = [(ev(), ev()) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for e0, e1 in pairs:
            step(e0, e1)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern_ms = sum(e0.elapsed_time(e1) for e0, e1 in pairs) / len(pairs)
        ms_per_step = wall * 1e3 / args.steps
        alg_bytes, alg_flops = prefill_algorithmic(T, H, d, C, True, True)
        achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
        traffic = measured_traffic(PREFILL_KERNEL)
        # MFMA share of peak on the algorithm's own flops, and the share that HBM
        # allows at this arithmetic intensity (the attainable roofline)
        mfma_frac = alg_flops / (kern_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS
        attainable = min(1.0, (alg_flops / alg_bytes) * HBM_PEAK_GBS * 1e9 /
                         (BF16_MFMA_PEAK_TFLOPS * 1e12))
        result.update({
            "value": T * args.steps / wall,
            "unit": "tokens/s",
            "ms_per_step": ms_per_step,
            "config": {"workload": "Ling-shaped KDA layer prefill: B=1, H=64, T=8192, "
                                   "d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 g/beta/state, "
                                   "zero initial state",
                       "global_batch": 1, "seq_len": T, "heads": H, "head_dim": d,
                       "chunk": C, "parallelism": "none (1 GPU)"},
            "roofline": {"bound": "hbm", "kernel": PREFILL_KERNELS, "achieved": achieved,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": traffic, "kernel_ms": kern_ms,
                         "algorithmic_bytes": alg_bytes},
            "mfma": {"algorithmic_tflops": alg_flops / (kern_ms * 1e-3) / 1e12,
                     "peak": BF16_MFMA_PEAK_TFLOPS,
                     "frac": mfma_frac,
                     "attainable_frac": attainable,
                     "attained_over_attainable": mfma_frac / attainable,
                     "rocprof_busy_frac": measured_mfma_busy(PREFILL_KERNEL),
                     "algorithmic_flops": alg_flops},
        })
        del q, k, v, g, beta, o, state
        if not args.no_cpu_baseline and args.only is None:
            result["cpu_baseline"] = cpu_baseline_run(inp)
        del inp
        torch.cuda.empty_cache()

    if args.only == "prefill_gate_proj" or (args.only is None and not args.no_decode):
        # the same layer with the gate prologue fused: bf16 decay projection f,
        # a_log = 0 and f = -N(3, 1), so that the decay has the layer's own
        # distribution; beta from fp32 logits
        inp = workloads.ling_prefill()
        T, H, d, C = inp.T, inp.H, inp.d, inp.chunk
        pr = workloads.gate_projections(T, H, d, dtype="bf16", g_mu=3.0, g_sigma=1.0,
                                        seed=1002)
        q, k, v, f, b, a_log = (x.to(dev) for x in (inp.q, inp.k, inp.v, pr.f, pr.b, pr.a_log))
        cu = inp.cu_seqlens.to(dev)
        state = torch.empty((1, H, d, d), dtype=torch.float32, device=dev)
        o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)

        def gstep(e0=None, e1=None):
            kda.kda_state_init(state)
            if e0 is not None:
                e0.record()
            kda.kda_prefill_chunked(q, k, v, f, b, cu_seqlens=cu, cu_seqlens_host=inp.cu_seqlens,
                                    chunk=C, initial_state=state, final_state=state, o=o,
                                    a_log=a_log)
            if e1 is not None:
                e1.record()

        for _ in range(args.warmup):
            gstep()
        torch.cuda.synchronize()
        gsteps = args.steps
        pairs = [(ev(), ev()) for _ in range(gsteps)]
        for e0_, e1_ in pairs:
            gstep(e0_, e1_)
        torch.cuda.synchronize()
        g_ms = sum(a.elapsed_time(b_) for a, b_ in pairs) / len(pairs)
        alg_bytes, _ = prefill_algorithmic(T, H, d, C, True, True, g_bytes=2)
        gbs = alg_bytes / (g_ms * 1e-3) / 1e9
        result["prefill_gate_proj"] = {
            "workload": "the Ling-shaped layer prefill with the gate prologue fused: bf16 decay "
                        "projection f [8192, 64, 128], a_log [64] = 0, fp32 beta logits",
            "ms_per_call": g_ms, "tokens_per_s": T / (g_ms * 1e-3),
            "roofline": {"bound": "hbm", "kernel": PREFILL_KERNELS, "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": None, "algorithmic_bytes": alg_bytes}}
        if args.only == "prefill_gate_proj":
            result.update({"value": T / (g_ms * 1e-3), "unit": "tokens/s",
                           "ms_per_step": g_ms})
        del q, k, v, f, b, a_log, o, state, inp, pr
        torch.cuda.empty_cache()

    if args.only == "prefill_out_gate" or (args.only is None and not args.no_decode):
        # the same layer with the output gate fused into the output stores: every
        # output multiplied by sigmoid(z), z a bf16 projection in o's layout
        inp = workloads.ling_prefill()
        T, H, d, C = inp.T, inp.H, inp.d, inp.chunk
        z = workloads.output_gate_projection(T, H, d, dtype="bf16", seed=1004)
        q, k, v, g, beta, zd = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, z))
        cu = inp.cu_seqlens.to(dev)
        state = torch.empty((1, H, d, d), dtype=torch.float32, device=dev)
        o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)

        def ostep(e0=None, e1=None):
            kda.kda_state_init(state)
            if e0 is not None:
                e0.record()
            kda.kda_prefill_chunked(q, k, v, g, beta, cu_seqlens=cu, cu_seqlens_host=inp.cu_seqlens,
                                    chunk=C, initial_state=state, final_state=state, o=o,
                                    out_gate=zd)
            if e1 is not None:
                e1.record()

        for _ in range(args.warmup):
            ostep()
        torch.cuda.synchronize()
        pairs = [(ev(), ev()) for _ in range(args.steps)]
        for e0_, e1_ in pairs:
            ostep(e0_, e1_)
        torch.cuda.synchronize()
        og_ms = sum(a.elapsed_time(b_) for a, b_ in pairs) / len(pairs)
        alg_bytes, _ = prefill_algorithmic(T, H, d, C, True, True)
        alg_bytes += T * H * d * 2  # the gate projection z, read once
        gbs = alg_bytes / (og_ms * 1e-3) / 1e9
        result["prefill_out_gate"] = {
            "workload": "the Ling-shaped layer prefill with the output gate fused: o * sigmoid(z), "
                        "z [8192, 64, 128] bf16",
            "ms_per_call": og_ms, "tokens_per_s": T / (og_ms * 1e-3),
            "roofline": {"bound": "hbm", "kernel": PREFILL_KERNELS, "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": None, "algorithmic_bytes": alg_bytes}}
        if args.only == "prefill_out_gate":
            result.update({"value": T / (og_ms * 1e-3), "unit": "tokens/s",
                           "ms_per_step": og_ms})
        del q, k, v, g, beta, zd, o, state, inp, z
        torch.cuda.empty_cache()

    B, H, d = 256, 64, 128  # the batched decode workload's shape
    nsteps = args.decode_steps if args.only is None else args.steps
    # untimed steps before each decode and conv timing: at least 50 in a full run
    # (decode, 50 steps after 5 warm-ups: 0.346 ms per step; 500 after 50: 0.332)
    dwarm = args.warmup if args.only is not None else max(args.warmup, 50)
    e0, e1 = ev(), ev()
    if args.only == "decode" or (args.only is None and not args.no_decode):
        inp = workloads.decode_batch()
        assert (inp.n_seqs, inp.H, inp.d) == (B, H, d)
        q, k, v, g, beta = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
        state = inp.S0.to(dev)
        o = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
        for _ in range(dwarm):
            kda.kda_decode_step(q, k, v, g, beta, state, o=o)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(nsteps):
            kda.kda_decode_step(q, k, v, g, beta, state, o=o)
        e1.record()
        torch.cuda.synchronize()
        step_ms = e0.elapsed_time(e1) / nsteps
        alg = decode_algorithmic(B, H, d)
        gbs = alg / (step_ms * 1e-3) / 1e9
        dec = {"workload": "batched decode step: B=256 sequences x H=64 heads, one token "
                           "each, fp32 128x128 states, bf16 q/k/v",
               "ms_per_step": step_ms, "tokens_per_s": B / (step_ms * 1e-3),
               "roofline": {"bound": "hbm", "kernel": DECODE_KERNEL, "achieved": gbs,
                            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                            "traffic": measured_traffic(DECODE_KERNEL),
                            "algorithmic_bytes": alg}}
        copy_gbs = copy_bandwidth(dev)
        dec["copy_kernel"] = {"achieved": copy_gbs, "unit": "GB/s",
                              "kernel": "copy16_kernel (kda_device_copy)",
                              "what": "16-byte non-temporal device copy of 1 GiB, read + "
                                      "written bytes per second"}
        dec["frac_of_copy"] = gbs / copy_gbs
        if not args.no_cpu_baseline and args.only is None:
            dec["cpu_single_thread"] = cpu_decode_single_thread(inp)
        if args.only == "decode":
            result.update({"value": B / (step_ms * 1e-3), "unit": "tokens/s",
                           "ms_per_step": step_ms})
        result["decode"] = dec
        # one decode step of all 63 KDA layers for one sequence reads and writes the
        # whole 63-layer state once: its time at the measured state bandwidth
        model_state = KDA_LAYERS * kda.kda_state_bytes(H, d, d)
        result["pages_context"] = {
            "kda_state_bytes_per_sequence_63_layers": model_state,
            "decode_state_us_per_token_63_layers": 2 * model_state / (gbs * 1e9) * 1e6,
            "decode_tokens_per_s_63_layers_state_bound": gbs * 1e9 / (2 * model_state),
            "kimi_linear_decode_claim": KIMI_LINEAR_DECODE_CLAIM,
        }
        del q, k, v, g, beta, state, o, inp

    if args.only == "decode_bf16_state" or (args.only is None and not args.no_decode):
        # the same step on states stored in bf16 (half the state bytes)
        inp = workloads.decode_batch()
        q, k, v, g, beta = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
        state = inp.S0.to(dev).to(torch.bfloat16)
        o = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
        for _ in range(dwarm):
            kda.kda_decode_step(q, k, v, g, beta, state, o=o)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(nsteps):
            kda.kda_decode_step(q, k, v, g, beta, state, o=o)
        e1.record()
        torch.cuda.synchronize()
        b16_ms = e0.elapsed_time(e1) / nsteps
        alg = decode_algorithmic(B, H, d, state_bytes=2)
        gbs = alg / (b16_ms * 1e-3) / 1e9
        result["decode_bf16_state"] = {
            "workload": "batched decode step as above with the states stored in bf16 (fp32 "
                        "arithmetic, rounded once per step when written)",
            "ms_per_step": b16_ms, "tokens_per_s": B / (b16_ms * 1e-3),
            "roofline": {"bound": "hbm", "kernel": DECODE_KERNEL + " (bf16 state)",
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(DECODE_BF16_KERNEL),
                         "algorithmic_bytes": alg}}
        if args.only == "decode_bf16_state":
            result.update({"value": B / (b16_ms * 1e-3), "unit": "tokens/s",
                           "ms_per_step": b16_ms})
        del q, k, v, g, beta, state, o, inp

    if args.only == "decode_tokens" or (args.only is None and not args.no_decode):
        # speculative-decoding verification: 4 tokens per sequence in one call
        n_tok = 4
        inp = workloads.recurrence_inputs([n_tok] * B, H=H, d=d, dtype="bf16", chunk=64,
                                          g_mu=2.0, g_sigma=0.5, s0_std=0.02, seed=1006)
        tk = lambda x: x.reshape((B, n_tok) + tuple(x.shape[1:])).to(dev).contiguous()
        q, k, v, g, beta = (tk(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
        state = inp.S0.to(dev)
        o = torch.empty((B, n_tok, H, d), dtype=torch.bfloat16, device=dev)
        for _ in range(dwarm):
            kda.kda_decode_tokens(q, k, v, g, beta, state, o=o)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(nsteps):
            kda.kda_decode_tokens(q, k, v, g, beta, state, o=o)
        e1.record()
        torch.cuda.synchronize()
        mtp_ms = e0.elapsed_time(e1) / nsteps
        alg = decode_algorithmic(B, H, d, n_tok)
        gbs = alg / (mtp_ms * 1e-3) / 1e9
        result["decode_tokens"] = {
            "workload": f"speculative-decoding verification: B={B} sequences x H={H} heads, "
                        f"{n_tok} tokens each per call, fp32 128x128 states, bf16 q/k/v",
            "ms_per_step": mtp_ms, "tokens_per_s": B * n_tok / (mtp_ms * 1e-3),
            "roofline": {"bound": "hbm", "kernel": DECODE_KERNEL + " (4 tokens per sequence)",
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(DECODE_TOKENS_KERNEL),
                         "algorithmic_bytes": alg}}
        if args.only == "decode_tokens":
            result.update({"value": B * n_tok / (mtp_ms * 1e-3), "unit": "tokens/s",
                           "ms_per_step": mtp_ms})
    if args.only == "conv" or (args.only is None and not args.no_decode):
        # the mixer's front end: width-4 causal conv of the q, k, v streams
        # (32768 x 8192 bf16 each), per-head L2 norm (128 channels) of q and k
        xs, ws = workloads.mixer_conv_streams()
        T, Cc = xs[0].shape
        xs = [x.to(dev) for x in xs]
        ws = [w.to(dev) for w in ws]
        ys = [torch.empty_like(x) for x in xs]
        cu_h = torch.tensor([0, T], dtype=torch.int32)
        cu_d = cu_h.to(dev)

        def front():
            for x, w, y, l2 in zip(xs, ws, ys, (128, 128, 0)):
                kda.kda_short_conv_prefill(x, w, cu_seqlens=cu_d, cu_seqlens_host=cu_h,
                                           l2_head_dim=l2, y=y)

        for _ in range(dwarm):
            front()
        torch.cuda.synchronize()
        csteps = max(1, min(nsteps, 100))
        e0.record()
        for _ in range(csteps):
            front()
        e1.record()
        torch.cuda.synchronize()
        conv_ms = e0.elapsed_time(e1) / csteps
        alg = 3 * (2 * T * Cc * 2 + Cc * 4 * 4)  # x read, y written, w read; per stream
        gbs = alg / (conv_ms * 1e-3) / 1e9
        result["conv_prefill"] = {
            "workload": f"mixer front end: width-4 causal conv of 3 streams [{T}, {Cc}] bf16, "
                        "per-head L2 norm (128 channels) of the q and k streams, one call each",
            "ms_per_step": conv_ms, "tokens_per_s": T / (conv_ms * 1e-3),
            "roofline": {"bound": "hbm", "kernel": "conv_prefill_wide_kernel (3 launches)",
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(CONV_KERNEL),
                         "algorithmic_bytes": alg}}
        if args.only == "conv":
            result.update({"value": T / (conv_ms * 1e-3), "unit": "tokens/s",
                           "ms_per_step": conv_ms})
        del xs, ws, ys
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
