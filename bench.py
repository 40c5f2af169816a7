#!/usr/bin/env python3
"""Benchmark of the decoder forward on one MI355X.

A step is one tfm_model_forward over a batch of synthetic token ids: embedding, the pre-norm
blocks (RMSNorm, QKV GEMM + RoPE, causal flash attention, out projection + residual, RMSNorm,
SwiGLU up GEMM, down projection + residual), final RMSNorm and the LM-head GEMM, with weights,
ids and the RoPE table already resident in HBM. Prints one JSON line.

Default workload: d_model 768, 12 layers, 12 heads of 64, d_ff 2048, vocabulary 50257, batch
8 x 1024 tokens, bf16 (--workload names the others).

Besides the step time it reports:
  step_kernels  every kernel family of the step timed INSIDE real steps: a second pass of the
                same number of steps runs with the library's launch trace on, so each launch is
                bracketed by HIP events on the launch stream. Per family: launches per step,
                average launch duration, time per step, algorithmic FLOPs and bytes per launch,
                and the fraction of its binding roofline (HBM when the algorithmic intensity is
                below the bf16 ridge of 312.5 flop/B, MFMA otherwise).
  roofline      that entry for the family with the most time per step (the dominant kernel),
                with its HBM traffic from the committed counter passes; roofline_lm_head the
                same for the LM head.
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same workload, with all
                host threads and with one.

With --counters it runs only what the hardware-counter passes need: a plain device copy of a
known size (the scale reference for the HBM byte counters), then two traced forward steps
(no warm-up) whose dispatches a counter summary attributes to kernel families by launch order;
it prints the launch labels of one step and exits without a JSON line. --attention-counters
likewise runs only ten launches of the step's causal attention. --train-only N and
--decode-only N run only the training leg or the decode leg (for kernel traces) and print
their mean step time.
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

PEAK_BF16 = 2.5e15       # dense bf16 MFMA FLOP/s (MI355X published)
PEAK_F32 = 157.3e12      # dense fp32 MFMA FLOP/s (MI355X published)
PEAK_HBM = 8.0e12        # HBM3E bytes/s (MI355X published)
COPY_BYTES = 1 << 30     # plain copy used to scale the HBM byte counters
METRIC = "decoder forward tokens/sec + attention/GEMM MFMA util, d768 L12 seq1024"

WORKLOADS = {"tiny": "TINY_F32", "small": "SMALL_BF16", "gpt2s": "GPT2S_BF16", "xl": "XL_BF16",
             "long_gqa": "LONG_GQA_BF16"}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_launches(fn, n: int, stream, graph: bool = True) -> float:
    """Average duration (ms) of fn() over n back-to-back launches on `stream` (captured once in
    a HIP graph and replayed when `graph`, so host launch overhead does not count)."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        start.record()
        g.replay()
        end.record()
        end.synchronize()
        return start.elapsed_time(end) / n
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(n):
            fn()
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "attention.hip", "elementwise.hip", "common.h", "api.cpp"):
        h.update(open(os.path.join(ROOT, "decoder_only_transformer_rmsnorm_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, label: str):
    """The committed counter summary of one kernel family (HBM bytes per launch from FETCH_SIZE
    and WRITE_SIZE), or None when absent or taken on different kernel sources."""
    try:
        d = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    except (OSError, ValueError):
        return None
    e = d.get(workload, {}).get(label)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e


def host_cpu() -> dict:
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"model": model, "nproc": usable, "cpu_count": os.cpu_count()}


def cpu_baseline(cfg, inputs, budget_s: float, threads: int):
    """The fp64 oracle on a bounded sample of the workload with `threads` OpenMP threads: whole
    sequences (every position, every logit) until about `budget_s` seconds have been spent, or
    a prefix of sequence 0 when one sequence alone would exceed it; tokens/s = tokens / wall
    time. Sequences are independent, so whole sequences give a fair rate; a prefix slightly
    overstates it (attention per token grows with the position)."""
    import numpy as np
    import oracle
    oracle.set_num_threads(threads)
    p0 = min(16, cfg.seq)          # probe; 64 tokens when 16 take under a tenth of the budget
    t0 = time.perf_counter()
    logits = oracle.model(cfg, inputs, ids=inputs.ids[:1, :p0])
    tp = time.perf_counter() - t0
    if tp < 0.1 * budget_s and cfg.seq > p0:
        p0 = min(64, cfg.seq)
        t0 = time.perf_counter()
        logits = oracle.model(cfg, inputs, ids=inputs.ids[:1, :p0])
        tp = time.perf_counter() - t0
    if tp > 0.4 * budget_s:      # the probe alone is a long enough sample
        assert np.isfinite(logits).all()
        sample = (f"sequence 0 of {cfg.batch}, positions 0..{p0 - 1} ({p0} tokens), all "
                  f"{cfg.vocab} logits per token")
        return {"value": round(p0 / tp, 2), "unit": "tokens/s", "cores": threads,
                "kind": "oracle", "sample": sample, "seconds": round(tp, 2)}
    if tp * (cfg.seq / p0) * 1.15 > budget_s:
        prefix = max(p0, int(p0 * budget_s / max(tp, 1e-9) / 1.15) // 16 * 16)
        t0 = time.perf_counter()
        logits = oracle.model(cfg, inputs, ids=inputs.ids[:1, :prefix])
        dt = time.perf_counter() - t0
        assert np.isfinite(logits).all()
        sample = (f"sequence 0 of {cfg.batch}, positions 0..{prefix - 1} ({prefix} tokens), all "
                  f"{cfg.vocab} logits per token")
        return {"value": round(prefix / dt, 2), "unit": "tokens/s", "cores": threads,
                "kind": "oracle", "sample": sample, "seconds": round(dt, 2)}
    done, dt = 0, 0.0
    while done < cfg.batch and dt < budget_s * 0.6:
        t0 = time.perf_counter()
        logits = oracle.model(cfg, inputs, ids=inputs.ids[done:done + 1])
        dt += time.perf_counter() - t0
        assert np.isfinite(logits).all()
        done += 1
    sample = (f"sequences 0..{done - 1} of {cfg.batch} ({done} x {cfg.seq} tokens), every "
              f"position and all {cfg.vocab} logits")
    return {"value": round(done * cfg.seq / dt, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": sample, "seconds": round(dt, 2)}


def rate_entry(label: str, w: dict, avg_ms: float, peak_mfma: float) -> dict:
    """A kernel family against its binding roofline (avg_ms: its launch duration in the step);
    both fractions are given."""
    s = avg_ms / 1e3
    e = {"kernel": label, "bound": w["bound"], "avg_launch_us": round(avg_ms * 1e3, 2),
         "flops_per_launch": int(w["flops"]), "bytes_per_launch": int(w["bytes"]),
         "TFLOP/s": round(w["flops"] / s / 1e12, 1), "GB/s": round(w["bytes"] / s / 1e9, 1),
         "frac_mfma": round(w["flops"] / s / peak_mfma, 4),
         "frac_hbm": round(w["bytes"] / s / PEAK_HBM, 4)}
    e["frac"] = e["frac_mfma"] if w["bound"] == "mfma" else e["frac_hbm"]
    return e


def roofline_of(entry: dict, peak_mfma: float, traffic) -> dict:
    mfma = entry["bound"] == "mfma"
    return {"bound": entry["bound"], "kernel": entry["kernel"],
            "achieved": entry["TFLOP/s"] if mfma else entry["GB/s"],
            "peak": round(peak_mfma / 1e12, 1) if mfma else PEAK_HBM / 1e9,
            "unit": "TFLOP/s" if mfma else "GB/s", "frac": entry["frac"],
            "traffic": traffic["bytes_per_launch"] if traffic else None,
            "per_launch": "algorithmic FLOPs" if mfma else "algorithmic HBM bytes",
            "flops_per_launch": entry["flops_per_launch"],
            "bytes_per_launch": entry["bytes_per_launch"],
            "avg_launch_us": entry["avg_launch_us"],
            "timing": "HIP events around every launch inside the traced steps on the launch "
                      "stream, less the trace's own cost per launch"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="gpt2s")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work per thread count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the sustained-rate probe, fused-loss, decode and training legs")
    ap.add_argument("--logits", choices=["bf16", "f32"], default="bf16")
    ap.add_argument("--dense-logits", action="store_true",
                    help="logits row stride = vocab (default: vocab rounded up to a multiple of "
                         "64 elements, so every logits row starts on a 128-byte line and no line "
                         "is shared by two output tiles)")
    ap.add_argument("--counters", action="store_true",
                    help="only a 1 GiB copy and 2 forward steps, for rocprofv3 --pmc passes")
    ap.add_argument("--attention-counters", action="store_true",
                    help="only 10 launches of the step's causal attention (random q, k, v of "
                         "the workload's shape), for rocprofv3 --pmc passes")
    ap.add_argument("--train-only", type=int, default=0, metavar="N",
                    help="only N training steps after 2 warm-up steps (for kernel traces of the "
                         "training step); prints the mean step time")
    ap.add_argument("--decode-only", type=int, default=0, metavar="N",
                    help="only a prefill of S - 24 positions and N decode steps after 3 warm-up "
                         "steps (for kernel traces of the decode step); prints the mean step time")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward shards by sequence with no exchange, "
              "and this benchmark reports the one-GPU rate only (run with --gpus 1).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from decoder_only_transformer_rmsnorm_amd import accounting, synth, tfm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    cfg = getattr(synth, WORKLOADS[args.workload])
    B, S, M = cfg.batch, cfg.seq, cfg.tokens
    bf16_model = cfg.dtype == "bf16"
    peak_mfma = PEAK_BF16 if bf16_model else PEAK_F32
    log(f"workload {cfg.name}: B={B} S={S} L={cfg.n_layers} d={cfg.d_model} "
        f"H={cfg.n_heads}/{cfg.n_kv_heads} dh={cfg.d_head} F={cfg.d_ff} V={cfg.vocab} {cfg.dtype}")
    t0 = time.perf_counter()
    inputs = synth.make_inputs(cfg, seed=0)
    dm = tfm.DeviceModel(inputs)
    log(f"inputs drawn and uploaded in {time.perf_counter() - t0:.1f} s")
    stream = torch.cuda.current_stream()
    logits_dtype = torch.float32 if (args.logits == "f32" or not bf16_model) else torch.bfloat16
    ld_logits = cfg.vocab if args.dense_logits else (cfg.vocab + 63) // 64 * 64
    logits = torch.empty((M, ld_logits), dtype=logits_dtype, device="cuda")
    lbytes = 4 if logits_dtype == torch.float32 else 2

    def step():
        dm.forward(logits=logits, ld_logits=ld_logits)

    if args.attention_counters:   # counter-pass mode: the step's attention alone
        qd, kvd = cfg.n_heads * cfg.d_head, cfg.n_kv_heads * cfg.d_head
        W = qd + 2 * kvd
        qkv = torch.randn((M, W), device="cuda").to(torch.bfloat16)
        o = torch.empty((M, qd), dtype=torch.bfloat16, device="cuda")
        for _ in range(10):
            tfm.tfm_causal_attention(
                qkv[:, :qd].view(B, S, qd), qkv[:, qd:qd + kvd].view(B, S, kvd),
                qkv[:, qd + kvd:].view(B, S, kvd), cfg.n_heads, cfg.n_kv_heads, cfg.d_head,
                o=o.view(B, S, qd), q_stride=W, kv_stride=W, o_stride=qd)
        torch.cuda.synchronize()
        log("attention counters run done: 10 launches")
        return 0
    if args.train_only > 0:   # kernel-trace mode: the training leg alone
        trn = tfm.Trainer(dm, lr=1e-4, weight_decay=0.1, max_norm=1.0)
        t_tg = tfm.next_token_targets(dm.ids)
        for _ in range(2):
            trn.step(dm.ids, t_tg)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.train_only):
            trn.step(dm.ids, t_tg)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.train_only
        print(json.dumps({"train_only": cfg.name, "steps": args.train_only,
                          "ms_per_step": round(ms, 3)}), flush=True)
        return 0
    if args.decode_only > 0:   # kernel-trace mode: the decode leg alone (as timed below)
        p0 = S - 24
        cache = dm.kv_cache(B, S)
        dm.prefill(cache, S, ids=dm.ids[:, :p0].contiguous(), logits=False)
        dlg = torch.empty((B, cfg.vocab), dtype=torch.bfloat16, device="cuda")
        dpos = torch.full((B,), p0, dtype=torch.int32, device="cuda")
        dtok = dm.ids[:, p0].contiguous()
        for _ in range(3):
            dm.decode(cache, S, dtok, dpos, logits=dlg)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.decode_only):
            dm.decode(cache, S, dtok, dpos, logits=dlg)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.decode_only
        print(json.dumps({"decode_only": cfg.name, "context": p0 + 1, "steps": args.decode_only,
                          "ms_per_step": round(ms, 4)}), flush=True)
        return 0
    if args.counters:
        src = torch.randn(COPY_BYTES // 4, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)              # reference: reads and writes exactly COPY_BYTES each
        torch.cuda.synchronize()
        with tfm.LaunchTrace(4096) as tr:
            step()
            step()
        labels = [l for l, _ in tr.records]
        per = len(labels) // 2
        assert labels[:per] == labels[per:]
        log(f"counters run done: copy {COPY_BYTES} B, 2 forward steps of {per} launches")
        print(json.dumps({"counters_run": cfg.name, "copy_bytes": COPY_BYTES,
                          "launch_labels_per_step": labels[:per]}), flush=True)
        return 0

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    dm.check_flags()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(logits[:: max(1, M // 64), : cfg.vocab]).all())

    log(f"timing {args.steps} steps")
    # one event per step boundary on the launch stream: the whole region gives ms_per_step,
    # the boundaries give the per-step median and minimum
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_med, ms_min = per[len(per) // 2], per[0]
    tok_s = M / (ms / 1e3)
    flops = accounting.forward_flops(cfg)
    log(f"{ms:.3f} ms/step, {tok_s / 1e6:.3f} M tokens/s, "
        f"{flops['total'] / (ms / 1e3) / 1e12:.1f} TFLOP/s end to end (wall {wall:.2f} s)")

    # ---- the same number of steps again with every launch bracketed by HIP events
    work = accounting.step_kernels(cfg, logits_bytes=lbytes)
    with tfm.LaunchTrace(args.steps * 80 * max(1, cfg.n_layers) + 16, stream) as tr:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    traced_ms = sum(t for _, t in tr.records) / args.steps
    agg = {}
    for label, t in tr.records:
        a = agg.setdefault(label, [0, 0.0])
        a[0] += 1
        a[1] += t
    # An event pair brackets a launch plus the gap before it, and recording the events costs
    # time of its own; that cost per launch is the traced step's excess over the untraced one
    # divided by the step's launches, and is taken off every launch's average.
    launches = len(tr.records) / args.steps
    trace_cost = max(0.0, traced_ms - ms) / launches
    step_kernels = {}
    for label, (n, tot) in agg.items():
        w = work.get(label)
        avg_gap = tot / n
        avg = max(avg_gap - trace_cost, 1e-6)
        e = rate_entry(label, w, avg, peak_mfma) if w else {"kernel": label,
                                                            "avg_launch_us": round(avg * 1e3, 2)}
        e["avg_launch_us_with_gap"] = round(avg_gap * 1e3, 2)
        e["launches_per_step"] = n // args.steps
        e["us_per_step"] = round(avg * n / args.steps * 1e3, 1)
        e["share_of_step"] = round(avg * n / args.steps / ms, 4)
        step_kernels[label] = e
    order = sorted(step_kernels, key=lambda k: -step_kernels[k]["us_per_step"])
    for k in order:
        e = step_kernels[k]
        log(f"in-step {k}: {e['launches_per_step']} x {e['avg_launch_us']} us = {e['us_per_step']} "
            f"us/step ({e['share_of_step']:.1%})" + (f", {e['bound']} frac {e['frac']}" if "frac" in e else ""))
    log(f"traced steps: {traced_ms:.3f} ms/step (untraced {ms:.3f}; trace cost "
        f"{trace_cost * 1e3:.2f} us per launch, taken off each launch)")
    dominant = next(k for k in order if k in work)
    roofline = roofline_of(step_kernels[dominant], peak_mfma,
                           traffic_from_profiles(cfg.name, dominant))
    roofline_lm = (roofline_of(step_kernels["gemm_lm_head"], peak_mfma,
                               traffic_from_profiles(cfg.name, "gemm_lm_head"))
                   if "gemm_lm_head" in step_kernels else None)
    gemm_labels = [k for k in step_kernels if k.startswith("gemm_")]
    att_labels = [k for k in step_kernels if k.startswith("attention")]
    def family(labels):
        f = sum(work[k]["flops"] * work[k]["launches"] for k in labels)
        t = sum(step_kernels[k]["us_per_step"] for k in labels) / 1e6
        return {"TFLOP/s": round(f / t / 1e12, 1), "frac_mfma": round(f / t / peak_mfma, 4),
                "us_per_step": round(t * 1e6, 1)} if t > 0 else None
    mfma_util = {"gemm": family(gemm_labels), "attention": family(att_labels)}
    rms = step_kernels.get("rmsnorm")
    rmsnorm_hbm = ({"GB/s": rms["GB/s"], "frac_hbm": rms["frac_hbm"],
                    "bytes_per_launch": rms["bytes_per_launch"],
                    "avg_launch_us": rms["avg_launch_us"]} if rms else None)

    extras = {}
    if not args.no_extras and bf16_model:
        # sustained matrix-core rate: a register-only loop of bf16 16x16x32 products on
        # pseudo-random operands, the second denominator beside the published dense peak
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        blocks, iters = 8 * cus, 20000
        sink = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
        L = tfm.lib()
        rate_ms = time_launches(lambda: L.tfm_mfma_rate(iters, blocks, sink.data_ptr(),
                                                        tfm._stream().pointer()), 3, stream)
        rate = blocks * 4 * iters * 8 * 2 * 16 * 16 * 32 / (rate_ms / 1e3)
        extras["mfma_sustained"] = {
            "TFLOP/s": round(rate / 1e12, 1), "frac_of_published": round(rate / PEAK_BF16, 4),
            "kernel": "register-only loop of 8 independent v_mfma_f32_16x16x32_bf16 per wave, "
                      "pseudo-random bf16 operands, 8 workgroups of 4 waves per CU"}
        log(f"sustained bf16 MFMA rate: {rate / 1e12:.1f} TFLOP/s ({rate / PEAK_BF16:.3f} of published)")
        roofline["frac_sustained"] = round(roofline["achieved"] / (rate / 1e12), 4) \
            if roofline["bound"] == "mfma" else None

        # forward ending in the fused LM head + next-token cross-entropy (no logits written)
        targets = tfm.next_token_targets(dm.ids)
        xloss = torch.empty(M, dtype=torch.float32, device="cuda")
        xmean = torch.empty(1, dtype=torch.float32, device="cuda")
        loss_ms = time_launches(lambda: dm.loss(targets, loss=xloss, mean=xmean), 10, stream,
                                graph=False)
        extras["loss_forward"] = {"ms_per_step": round(loss_ms, 4),
                                  "tokens_per_s": round(M / (loss_ms / 1e3), 1),
                                  "mean_loss": round(float(xmean.item()), 4)}
        log(f"forward with fused loss: {loss_ms:.3f} ms/step, {M / (loss_ms / 1e3) / 1e6:.3f} M tokens/s")

        if cfg.name == synth.GPT2S_BF16.name:
            # KV-cache decode: prefill all but the last 24 positions, then time one-token steps
            # at that context (each step rewrites the same slot: identical work every step)
            cache_seq = S
            p0 = S - 24
            cache = dm.kv_cache(B, cache_seq)
            dm.prefill(cache, cache_seq, ids=dm.ids[:, :p0].contiguous(), logits=False)
            dec_logits = torch.empty((B, cfg.vocab), dtype=torch.bfloat16, device="cuda")
            dec_pos = torch.full((B,), p0, dtype=torch.int32, device="cuda")
            dec_tok = dm.ids[:, p0].contiguous()
            step_fn = lambda: dm.decode(cache, cache_seq, dec_tok, dec_pos, logits=dec_logits)
            eager_ms = time_launches(step_fn, 20, stream, graph=False)
            graph_ms = time_launches(step_fn, 20, stream, graph=True)
            dm.check_decode_flags()
            dbytes = accounting.decode_bytes(cfg, B, p0 + 1)
            extras["decode"] = {
                "batch": B, "context": p0 + 1, "cache_seq": cache_seq,
                "ms_per_step_graph": round(graph_ms, 4), "ms_per_step_eager": round(eager_ms, 4),
                "tokens_per_s": round(B / (graph_ms / 1e3), 1),
                "hbm_bytes_per_step": int(dbytes["total"]),
                "GB/s": round(dbytes["total"] / (graph_ms / 1e3) / 1e9, 1),
                "frac_hbm": round(dbytes["total"] / (graph_ms / 1e3) / PEAK_HBM, 4)}
            log(f"decode B={B} context {p0 + 1}: {graph_ms * 1e3:.1f} us/step in a graph "
                f"({eager_ms * 1e3:.1f} eager), {extras['decode']['GB/s']} GB/s algorithmic")
            del cache

            # training step on the same batch: forward keeping activations, backward,
            # global-norm clipping and AdamW (it rewrites the weights, so it runs last)
            trn = tfm.Trainer(dm, lr=1e-4, weight_decay=0.1, max_norm=1.0)
            t_tg = tfm.next_token_targets(dm.ids)
            loss0 = float(trn.step(dm.ids, t_tg).item())
            train_ms = time_launches(lambda: trn.step(dm.ids, t_tg), 5, stream, graph=False)
            fw = flops["total"]
            extras["train_step"] = {
                "ms_per_step": round(train_ms, 3), "tokens_per_s": round(M / (train_ms / 1e3), 1),
                "loss_first_step": round(loss0, 4),
                "model_TFLOP/s": round(3 * fw / (train_ms / 1e3) / 1e12, 1),
                "flops_note": "3 x forward (causal) per step"}
            log(f"training step: {train_ms:.2f} ms, {M / (train_ms / 1e3) / 1e3:.1f} k tokens/s")
            del trn

    cpu = None
    if not args.no_cpu_baseline:
        host = host_cpu()
        log(f"cpu baseline: oracle on {host['nproc']} usable threads ({host['model']}), "
            f"budget {args.cpu_budget:.0f} s per thread count")
        cpu = cpu_baseline(cfg, inputs, args.cpu_budget, host["nproc"])
        one = cpu_baseline(cfg, inputs, args.cpu_budget, 1)
        cpu["sample"] += f", fp64 oracle with {host['nproc']} OpenMP threads"
        cpu["host"] = host
        cpu["one_thread"] = {"value": one["value"], "sample": one["sample"],
                             "seconds": one["seconds"]}
        log(f"cpu baseline {cpu['value']:.2f} tokens/s on {host['nproc']} threads "
            f"({cpu['sample']}); {one['value']:.2f} tokens/s on 1 thread ({one['sample']})")

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_median": round(ms_med, 4), "ms_min": round(ms_min, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded uniform ids, N(0,0.02) weights)",
        "config": {"workload": cfg.name, "batch": B, "seq_len": S, "n_layers": cfg.n_layers,
                   "d_model": cfg.d_model, "n_heads": cfg.n_heads, "n_kv_heads": cfg.n_kv_heads,
                   "d_head": cfg.d_head, "d_ff": cfg.d_ff, "vocab": cfg.vocab,
                   "logits_dtype": "f32" if lbytes == 4 else "bf16", "ld_logits": ld_logits,
                   "parallelism": "single GPU"},
        "end_to_end": {"flops_per_step_causal": int(flops["total"]),
                       "TFLOP/s": round(flops["total"] / (ms / 1e3) / 1e12, 1),
                       "frac_mfma": round(flops["total"] / (ms / 1e3) / peak_mfma, 4),
                       "frac_mfma_sustained": (round(flops["total"] / (ms / 1e3) / 1e12
                                                     / extras["mfma_sustained"]["TFLOP/s"], 4)
                                               if "mfma_sustained" in extras else None)},
        "roofline": roofline,
        "roofline_lm_head": roofline_lm,
        "traced_ms_per_step": round(traced_ms, 4),
        "trace_cost_us_per_launch": round(trace_cost * 1e3, 3),
        "step_kernels": step_kernels,
        "mfma_util": mfma_util,
        "rmsnorm_hbm": rmsnorm_hbm,
        **extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
