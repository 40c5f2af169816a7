#!/usr/bin/env python3
"""Benchmark of the decoder forward on one MI355X.

A step is one tfm_model_forward over a batch of synthetic token ids: embedding, 12 pre-norm
blocks (RMSNorm, QKV GEMM + RoPE, causal flash attention, out projection + residual,
RMSNorm, SwiGLU up GEMM, down projection + residual), final RMSNorm and the LM-head GEMM,
with weights, ids and the RoPE table already resident in HBM. Prints one JSON line.

Besides the step time it reports:
  roofline      the dominant kernel (the LM-head GEMM) timed alone through its entry point
                on the same stream with HIP events: algorithmic FLOPs per launch divided by
                the average launch duration, against the bf16 dense MFMA peak.
  kernels       the same measurement for each kernel family of the step.
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same workload.

With --counters it runs only what the hardware-counter passes need: one plain device copy of
a known size (the scale reference for the HBM byte counters) and a few launches of the
LM-head GEMM, then exits without a JSON line; --attention-counters likewise runs only ten
launches of the step's attention.
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
PEAK_HBM = 8.0e12        # HBM3E bytes/s (MI355X published)
COPY_BYTES = 1 << 30     # plain copy used to scale the HBM byte counters
METRIC = "decoder forward tokens/sec + attention/GEMM MFMA util, d768 L12 seq1024"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_launches(fn, n: int, stream, graph: bool = True) -> float:
    """Average duration (ms) of fn() over n back-to-back launches on `stream`.

    With `graph`, the n launches are captured once in a HIP graph and the replay is timed,
    so host-side launch overhead (Python, ctypes) does not inflate short kernels."""
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
    for f in ("gemm.hip", "common.h"):
        h.update(open(os.path.join(ROOT, "decoder_only_transformer_rmsnorm_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key: str):
    """The committed PMC summary entry of the dominant kernel (HBM bytes per launch, kernel
    name), or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e


def cpu_baseline(cfg, inputs, budget_s: float):
    """The fp64 oracle on a bounded sample of the workload: whole sequences (every position,
    every logit), one after another, until about `budget_s` seconds of CPU work have been
    spent; tokens/s = tokens / wall time. Sequences are independent, so this is a fair rate.
    If one sequence alone would exceed the budget, a prefix of sequence 0 is timed instead."""
    import numpy as np
    import oracle
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    oracle.model(cfg, inputs, ids=inputs.ids[:1, :64])
    t64 = time.perf_counter() - t0
    if t64 * (cfg.seq / 64) * 1.15 > budget_s:
        prefix = max(64, int(64 * budget_s / max(t64, 1e-9) / 1.15) // 64 * 64)
        t0 = time.perf_counter()
        logits = oracle.model(cfg, inputs, ids=inputs.ids[:1, :prefix])
        dt = time.perf_counter() - t0
        assert np.isfinite(logits).all()
        sample = (f"sequence 0 of {cfg.batch}, positions 0..{prefix - 1} ({prefix} tokens), all "
                  f"{cfg.vocab} logits per token, fp64 oracle with {threads} OpenMP threads")
        return {"value": prefix / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": sample, "seconds": round(dt, 2)}
    done, dt = 0, 0.0
    while done < cfg.batch and dt < budget_s * 0.6:
        t0 = time.perf_counter()
        logits = oracle.model(cfg, inputs, ids=inputs.ids[done:done + 1])
        dt += time.perf_counter() - t0
        assert np.isfinite(logits).all()
        done += 1
    sample = (f"sequences 0..{done - 1} of {cfg.batch} ({done} x {cfg.seq} tokens), every position "
              f"and all {cfg.vocab} logits, fp64 oracle with {threads} OpenMP threads")
    return {"value": done * cfg.seq / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel timing")
    ap.add_argument("--logits", choices=["bf16", "f32"], default="bf16")
    ap.add_argument("--dense-logits", action="store_true",
                    help="logits row stride = vocab (default: vocab rounded up to a multiple of "
                         "64 elements, so every logits row starts on a 128-byte line and no line "
                         "is shared by two output tiles)")
    ap.add_argument("--counters", action="store_true",
                    help="only a 1 GiB copy and 3 LM-head launches, for rocprofv3 --pmc passes")
    ap.add_argument("--attention-counters", action="store_true",
                    help="only 10 launches of the step's causal attention (random q, k, v of "
                         "the workload's shape), for rocprofv3 --pmc passes")
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
    cfg = synth.GPT2S_BF16
    B, S, M = cfg.batch, cfg.seq, cfg.tokens
    log(f"workload {cfg.name}: B={B} S={S} L={cfg.n_layers} d={cfg.d_model} V={cfg.vocab}")
    inputs = synth.make_inputs(cfg, seed=0)
    dm = tfm.DeviceModel(inputs)
    stream = torch.cuda.current_stream()
    logits_dtype = torch.float32 if args.logits == "f32" else torch.bfloat16
    ld_logits = cfg.vocab if args.dense_logits else (cfg.vocab + 63) // 64 * 64
    logits = torch.empty((M, ld_logits), dtype=logits_dtype, device="cuda")

    def step():
        dm.forward(logits=logits, ld_logits=ld_logits)

    if args.attention_counters:
        qd = cfg.n_heads * cfg.d_head
        qkv = torch.randn((M, 3 * qd), device="cuda").to(torch.bfloat16)
        o = torch.empty((M, qd), dtype=torch.bfloat16, device="cuda")
        for _ in range(10):
            tfm.tfm_causal_attention(
                qkv[:, :qd].view(B, S, qd), qkv[:, qd:2 * qd].view(B, S, qd),
                qkv[:, 2 * qd:].view(B, S, qd), cfg.n_heads, cfg.n_kv_heads, cfg.d_head,
                o=o.view(B, S, qd), q_stride=3 * qd, kv_stride=3 * qd, o_stride=qd)
        torch.cuda.synchronize()
        log("attention counters run done: 10 launches")
        return 0

    if args.counters:
        xn = torch.randn((M, cfg.d_model), device="cuda").to(torch.bfloat16)
        src = torch.randn(COPY_BYTES // 4, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)              # reference: reads and writes exactly COPY_BYTES each
        torch.cuda.synchronize()
        for _ in range(3):
            tfm.tfm_linear(xn, dm.lm_head, y=logits)
        torch.cuda.synchronize()
        log(f"counters run done: copy {COPY_BYTES} B, 3 LM-head launches")
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

    # ---- the sustained matrix-core rate: a register-only loop of bf16 16x16x32 products on
    #      pseudo-random operands (tfm_mfma_rate), the second denominator beside the published
    #      dense peak, which assumes the top clock the chip does not hold under random data
    mfma_sustained = None
    if not args.no_kernels:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        blocks, iters = 8 * cus, 20000
        sink = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
        L = tfm.lib()
        rate_ms = time_launches(lambda: L.tfm_mfma_rate(iters, blocks, sink.data_ptr(), tfm._stream()),
                                3, stream)
        rate = blocks * 4 * iters * 8 * 2 * 16 * 16 * 32 / (rate_ms / 1e3)
        mfma_sustained = {"TFLOP/s": round(rate / 1e12, 1), "frac_of_published": round(rate / PEAK_BF16, 4),
                          "ms": round(rate_ms, 3), "workgroups": blocks, "iterations": iters,
                          "kernel": "register-only loop of 8 independent v_mfma_f32_16x16x32_bf16 "
                                    "per wave, pseudo-random bf16 operands"}
        log(f"sustained bf16 MFMA rate: {rate / 1e12:.1f} TFLOP/s ({rate / PEAK_BF16:.3f} of published)")

    # ---- per-kernel timing through each entry point, same shapes as inside the step
    kernels = {}
    roofline = None
    loss_forward = None
    mfma_util = None
    decode = None
    if not args.no_kernels:
        D, F, V = cfg.d_model, cfg.d_ff, cfg.vocab
        qd = cfg.n_heads * cfg.d_head
        bf = torch.bfloat16
        gen = torch.Generator(device="cuda").manual_seed(0)
        xres = torch.randn((M, D), device="cuda", generator=gen)
        xn = torch.randn((M, D), device="cuda", generator=gen).to(bf)
        L0 = dm.layers[0]
        qkv = torch.randn((M, qd * 3), device="cuda", generator=gen).to(bf)
        o = torch.empty((M, qd), dtype=bf, device="cuda")
        u = torch.randn((M, F), device="cuda", generator=gen).to(bf)
        ws_ffn = torch.empty(tfm.lib().tfm_swiglu_workspace_bytes(M, F, 1), dtype=torch.uint8, device="cuda")
        xout = torch.empty((M, D), device="cuda")
        n = args.kernel_reps
        flops_gemm = lambda N, K: 2.0 * M * N * K

        def rec(name, ms_k, work, bound, unit_work):
            if bound == "hbm":
                ach = work / (ms_k / 1e3)
                kernels[name] = {"ms": round(ms_k, 4), "GB/s": round(ach / 1e9, 1),
                                 "frac_hbm": round(ach / PEAK_HBM, 4), "bytes": int(work)}
            else:
                ach = work / (ms_k / 1e3)
                kernels[name] = {"ms": round(ms_k, 4), "TFLOP/s": round(ach / 1e12, 1),
                                 "frac_mfma": round(ach / PEAK_BF16, 4), "flops": int(work)}
            log(f"kernel {name}: {ms_k * 1e3:.1f} us, {kernels[name]}")

        rec("rmsnorm", time_launches(lambda: tfm.tfm_rmsnorm(xres, L0["g_attn"], cfg.eps, y=xn), n, stream),
            accounting.rmsnorm_bytes(M, D, 4, 2), "hbm", None)
        qkv_out = torch.empty((B, S, 3 * qd), dtype=bf, device="cuda")
        rec("gemm_qkv_rope", time_launches(lambda: tfm.tfm_qkv_rope(
            xn.view(B, S, D), L0["wq"], L0["wk"], L0["wv"], cfg.n_heads, cfg.n_kv_heads, cfg.d_head,
            dm.cos_sin, dm.max_seq, qkv=qkv_out), n, stream), flops_gemm(3 * qd, D), "mfma", None)
        att_flops = accounting.forward_flops(cfg)["attn"] / cfg.n_layers
        rec("attention", time_launches(lambda: tfm.tfm_causal_attention(
            qkv[:, :qd].view(B, S, qd), qkv[:, qd:2 * qd].view(B, S, qd), qkv[:, 2 * qd:].view(B, S, qd),
            cfg.n_heads, cfg.n_kv_heads, cfg.d_head, o=o.view(B, S, qd),
            q_stride=3 * qd, kv_stride=3 * qd, o_stride=qd), n, stream), att_flops, "mfma", None)
        # sliding-window attention over the same q, k, v (band of 256 keys per query)
        win = 256
        rec(f"attention_window{win}", time_launches(lambda: tfm.tfm_sliding_window_attention(
            qkv[:, :qd].view(B, S, qd), qkv[:, qd:2 * qd].view(B, S, qd), qkv[:, 2 * qd:].view(B, S, qd),
            cfg.n_heads, cfg.n_kv_heads, cfg.d_head, win, o=o.view(B, S, qd),
            q_stride=3 * qd, kv_stride=3 * qd, o_stride=qd), n, stream),
            accounting.attention_flops(B, S, cfg.n_heads, cfg.d_head, win), "mfma", None)
        rec("gemm_out_residual", time_launches(lambda: tfm.tfm_linear(o, L0["wo"], residual=xres, y=xres), n, stream),
            flops_gemm(D, qd), "mfma", None)
        rec("swiglu_ffn", time_launches(lambda: tfm.lib().tfm_swiglu_ffn(
            xn.data_ptr(), L0["w1"].data_ptr(), L0["w3"].data_ptr(), L0["w2"].data_ptr(), xres.data_ptr(),
            xout.data_ptr(), M, D, F, 1, ws_ffn.data_ptr(), ws_ffn.numel(), tfm._stream()), n, stream),
            flops_gemm(2 * F, D) + flops_gemm(D, F), "mfma", None)
        rec("gemm_down_residual", time_launches(lambda: tfm.tfm_linear(u, L0["w2"], residual=xres, y=xres), n, stream),
            flops_gemm(D, F), "mfma", None)
        lm_ms = time_launches(lambda: tfm.tfm_linear(xn, dm.lm_head, y=logits), n, stream)
        rec("gemm_lm_head", lm_ms, flops_gemm(V, D), "mfma", None)
        lm_flops = flops_gemm(V, D)
        ach = lm_flops / (lm_ms / 1e3) / 1e12
        prof = traffic_from_profiles("gemm_lm_head")
        roofline = {"bound": "mfma",
                    "kernel": (prof["kernel"] if prof else "gemm_bf16_kernel, plain-store epilogue")
                              + f" (LM head, M={M} N={V} K={D}, logits row stride {ld_logits})",
                    "achieved": round(ach, 1), "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                    "frac": round(ach * 1e12 / PEAK_BF16, 4), "flops_per_launch": int(lm_flops),
                    "avg_launch_ms": round(lm_ms, 4),
                    "traffic": prof["bytes_per_launch"] if prof else None}
        if mfma_sustained:
            roofline["peak_sustained"] = mfma_sustained["TFLOP/s"]
            roofline["frac_sustained"] = round(ach / mfma_sustained["TFLOP/s"], 4)

        # fused LM head + next-token cross-entropy (no logits written), and the whole forward
        # ending in it
        targets = tfm.next_token_targets(dm.ids)
        xloss = torch.empty(M, dtype=torch.float32, device="cuda")
        xmean = torch.empty(1, dtype=torch.float32, device="cuda")
        rec("lm_head_xent", time_launches(lambda: tfm.tfm_lm_head_xent(
            xn, dm.lm_head, targets.view(-1), loss=xloss, mean=xmean), n, stream),
            flops_gemm(V, D), "mfma", None)
        loss_ms = time_launches(lambda: dm.loss(targets, loss=xloss, mean=xmean), max(2, n // 4),
                                stream, graph=False)
        loss_forward = {"ms_per_step": round(loss_ms, 4), "tokens_per_s": round(M / (loss_ms / 1e3), 1),
                        "mean_loss": round(float(xmean.item()), 4)}
        log(f"forward with fused loss: {loss_ms:.3f} ms/step, {M / (loss_ms / 1e3) / 1e6:.3f} M tokens/s")

        # KV-cache decode: prefill all but the last 24 positions, then time one-token steps at
        # that context (each step rewrites the same slot, so every step does identical work)
        cache_seq = S
        p0 = S - 24
        cache = dm.kv_cache(B, cache_seq)
        dm.prefill(cache, cache_seq, ids=dm.ids[:, :p0].contiguous(), logits=False)
        dec_logits = torch.empty((B, V), dtype=bf, device="cuda")
        dec_pos = torch.full((B,), p0, dtype=torch.int32, device="cuda")
        dec_tok = dm.ids[:, p0].contiguous()
        step_fn = lambda: dm.decode(cache, cache_seq, dec_tok, dec_pos, logits=dec_logits)
        eager_ms = time_launches(step_fn, 20, stream, graph=False)
        graph_ms = time_launches(step_fn, 20, stream, graph=True)
        dm.check_decode_flags()
        dbytes = accounting.decode_bytes(cfg, B, p0 + 1)
        decode = {"batch": B, "context": p0 + 1, "cache_seq": cache_seq,
                  "ms_per_step_graph": round(graph_ms, 4), "ms_per_step_eager": round(eager_ms, 4),
                  "tokens_per_s": round(B / (graph_ms / 1e3), 1),
                  "hbm_bytes_per_step": int(dbytes["total"]),
                  "GB/s": round(dbytes["total"] / (graph_ms / 1e3) / 1e9, 1),
                  "frac_hbm": round(dbytes["total"] / (graph_ms / 1e3) / PEAK_HBM, 4)}
        log(f"decode B={B} context {p0 + 1}: {graph_ms * 1e3:.1f} us/step in a graph "
            f"({eager_ms * 1e3:.1f} eager), {decode['GB/s']} GB/s algorithmic")
        del cache

        # MFMA utilisation of the GEMM and attention kernels over one step
        L_ = cfg.n_layers
        gemm_f = L_ * (flops_gemm(3 * qd, D) + flops_gemm(D, qd) + flops_gemm(2 * F, D)
                       + flops_gemm(D, F)) + flops_gemm(V, D)
        gemm_ms = L_ * (kernels["gemm_qkv_rope"]["ms"] + kernels["gemm_out_residual"]["ms"]
                        + kernels["swiglu_ffn"]["ms"]) + kernels["gemm_lm_head"]["ms"]
        mfma_util = {"gemm": round(gemm_f / (gemm_ms / 1e3) / PEAK_BF16, 4),
                     "attention": kernels["attention"]["frac_mfma"]}

    train = None
    if not args.no_kernels:
        # training step on the same batch: forward keeping activations, backward, global-norm
        # clipping and AdamW (it rewrites the weights, so it runs after every other leg)
        tr = tfm.Trainer(dm, lr=1e-4, weight_decay=0.1, max_norm=1.0)
        t_tg = tfm.next_token_targets(dm.ids)
        loss0 = float(tr.step(dm.ids, t_tg).item())
        train_ms = time_launches(lambda: tr.step(dm.ids, t_tg), 5, stream, graph=False)
        fw = accounting.forward_flops(cfg)["total"]
        train = {"ms_per_step": round(train_ms, 3), "tokens_per_s": round(M / (train_ms / 1e3), 1),
                 "loss_first_step": round(loss0, 4),
                 "model_TFLOP/s": round(3 * fw / (train_ms / 1e3) / 1e12, 1),
                 "flops_note": "3 x forward (causal) per step"}
        log(f"training step: {train_ms:.2f} ms, {M / (train_ms / 1e3) / 1e3:.1f} k tokens/s")
        del tr

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle, budget {args.cpu_budget:.0f} s")
        cpu = cpu_baseline(cfg, inputs, args.cpu_budget)
        log(f"cpu baseline {cpu['value']:.2f} tokens/s ({cpu['sample']}, {cpu['seconds']} s)")

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_median": round(ms_med, 4), "ms_min": round(ms_min, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded uniform ids, N(0,0.02) weights)",
        "config": {"workload": cfg.name, "batch": B, "seq_len": S, "n_layers": cfg.n_layers,
                   "d_model": cfg.d_model, "n_heads": cfg.n_heads, "d_ff": cfg.d_ff,
                   "vocab": cfg.vocab, "logits_dtype": args.logits, "ld_logits": ld_logits,
                   "parallelism": "single GPU"},
        "end_to_end": {"flops_per_step_causal": int(flops["total"]),
                       "TFLOP/s": round(flops["total"] / (ms / 1e3) / 1e12, 1),
                       "frac_mfma": round(flops["total"] / (ms / 1e3) / PEAK_BF16, 4),
                       "frac_mfma_sustained": (round(flops["total"] / (ms / 1e3) / 1e12
                                                     / mfma_sustained["TFLOP/s"], 4)
                                               if mfma_sustained else None)},
        "mfma_sustained": mfma_sustained,
        "roofline": roofline,
        "mfma_util": mfma_util,
        "kernels": kernels,
        "loss_forward": loss_forward,
        "decode": decode,
        "train_step": train,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
