"""Benchmark of the MI355X decoder layer (one GPU).

Step = one causal prefill of the LLaMA-3-8B-shaped layer (d 4096, 32 query
heads, 8 KV heads, I 14336, B 1, S 8192, bf16, fp32 accumulation) through the
C ABI, on synthetic seeded inputs already resident in HBM.  The same run also
times 128 consecutive batched decode steps of that layer (B 64, paged cache
pre-filled at context lengths drawn from U[512, 8192]), reported under
"decode".  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--decode-steps N] [--no-cpu-baseline]
                    [--prefill-workload NAME] [--decode-workload NAME] [--stack-layers N]

The workload options time the other shapes with the same step definition:
the LLaMA-2-7B (MHA) and LLaMA-3-70B layers, and the GQA ratio sweep (MQA at
the 8B shape, the LLaMA-3-405B layer); the defaults are the 8B jobs above.  --stack-layers N times N such layers
(each with its own weights, over one N-layer paged cache) plus the final
RMSNorm as the step instead of one layer.
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

METRIC = "layer prefill tokens/s + decode µs/step, LLaMA-3-8B shape; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_llama3_8b_prefill_decode.md")


def traffic_record(kernel: str):
    """HBM traffic of `kernel` from the committed rocprofv3 counter summary, or
    None when there is none or the kernel's sources changed since it was taken."""
    import hashlib
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for line in lines:
        parts = line.split()
        if not parts or parts[0] != "traffic-record":
            continue
        rec = dict(p.split("=", 1) for p in parts[1:])
        if rec.get("kernel") != kernel:
            continue
        h = hashlib.sha256()
        try:
            for src in rec["sources"].split(","):
                h.update(open(os.path.join(ROOT, src), "rb").read())
        except OSError:
            return None
        return rec if h.hexdigest() == rec.get("sha256") else None
    return None


def prefill_flops(w) -> dict:
    """Algorithmic flops per kernel family of one prefill (causal pairs only)."""
    T = w.batch * w.seq_len
    d, I, H, G, D = w.hidden_size, w.intermediate_size, w.num_attention_heads, w.num_key_value_heads, w.head_dim
    pairs = w.batch * w.seq_len * (w.seq_len + 1) // 2
    return {"gemm_qkv_rope": 2 * T * d * (H + 2 * G) * D,
            "attn_prefill": 4 * D * H * pairs,
            "gemm_o_resid": 2 * T * H * D * d,
            "gemm_gate_up_swiglu": 4 * T * d * I,
            "gemm_down_resid": 2 * T * I * d}


def make_model(args, L, synth, w, max_pos):
    """The layer, or (--stack-layers N > 1) a stack of N layers with their own
    weights and the final RMSNorm; returns (runner, [layer handles])."""
    nl = args.stack_layers
    layers = []
    for l in range(nl):
        ws = synth.layer_weights(w, layer=l)
        layers.append(L.DecoderLayer(w.config_dict(), ws, "bf16", max_pos))
        del ws
    if nl == 1:
        return layers[0], layers
    return L.DecoderStack(layers, synth.final_norm_weight(w)), layers


def make_cache(L, model, layers, nb, batch, order=None):
    if len(layers) == 1:
        return L.PagedKVCache(model, nb, batch, block_order=order)
    return model.cache(nb, batch, block_order=order)


def profile_all(L, layers, on):
    for layer in layers:
        L.llama_layer_profile_enable(layer.handle, on)


def profile_sum(L, layers):
    """Per-kernel (launches, total ms) summed over the layers."""
    tot = {}
    for layer in layers:
        for name, (n, ms) in L.llama_layer_profile_read(layer.handle, reset=True).items():
            a, b = tot.get(name, (0, 0.0))
            tot[name] = (a + n, b + ms)
    return tot


def run_prefill(args, torch, L, synth):
    w = synth.PREFILL_JOBS[args.prefill_workload]
    nl = args.stack_layers
    log(f"[bench] prefill workload {w.name}" + (f", stack of {nl} layers" if nl > 1 else "") + ": generating weights")
    model, layers = make_model(args, L, synth, w, w.positions_needed())
    x = synth.layer_input(w).cuda()
    cache = make_cache(L, model, layers, w.batch * ((w.seq_len + 15) // 16), w.batch)
    out = torch.empty((w.batch, w.seq_len, w.hidden_size), dtype=torch.bfloat16, device="cuda")

    def step():
        sids = [cache.add_seq() for _ in range(w.batch)]
        model.prefill(cache, sids, x, out_dtype="bf16", out=out)
        for s in sids:
            cache.free_seq(s)

    for _ in range(args.warmup):
        step()
    # timed steps without per-kernel events ...
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    # ... then the same number of steps again with HIP events around every
    # launch on the layer's stream, for the per-kernel breakdown
    profile_all(L, layers, True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    prof = profile_sum(L, layers)
    profile_all(L, layers, False)
    ms_prof = (t2 - t1) * 1e3 / args.steps
    flops = {k: v * nl for k, v in prefill_flops(w).items()}
    kern = {}
    for name, (n, tot) in prof.items():
        avg = tot / n
        kern[name] = {"avg_ms": round(avg, 4), "launches": n}
        if name in flops:
            kern[name]["tflops"] = round(flops[name] / nl / (avg * 1e-3) / 1e12, 1)  # per launch
    dom = "gemm_gate_up_swiglu"
    dom_ms = prof[dom][1] / prof[dom][0]
    ach = flops[dom] / nl / (dom_ms * 1e-3) / 1e12
    total_flops = sum(flops.values())
    rec = traffic_record(dom)
    traffic = int(rec["bytes_per_launch"]) if rec and "bytes_per_launch" in rec else None
    log(f"[bench] prefill {ms:.3f} ms/step ({ms_prof:.3f} with per-kernel events), "
        f"layer {total_flops / ms / 1e9:.1f} TFLOP/s")
    layer_ach = total_flops / (ms * 1e-3) / 1e12
    res = {
        "tokens_per_s": w.batch * w.seq_len / (ms * 1e-3), "ms": ms, "ms_profiled": ms_prof, "kernels": kern,
        "layer_tflops": layer_ach,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": flops[dom] // nl, "avg_launch_ms": round(dom_ms, 4)},
        # the whole layer against the same peak: every kernel's algorithmic flops
        # over the wall-clock step time (norms and launch gaps included)
        "layer_roofline": {"bound": "mfma", "achieved": round(layer_ach, 1), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(layer_ach / PEAK_BF16_TFLOPS, 4),
                           "flops_per_step": total_flops},
    }
    cache.close()
    model.close()
    for layer in layers:
        layer.close()
    return w, res


def run_other_workloads(args, torch, L, synth):
    """Quick timings of the other workload definitions, so that their numbers
    reach the result line: the tiny fp32 layer's prefill and decode-step
    latency, and the LLaMA-7B and LLaMA-3-70B layer prefills (wall clock
    around back-to-back calls with inputs in HBM, no per-kernel events)."""
    out = {}

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    # tiny fp32 layer: B 1, S 64 prefill, then decode steps against its cache
    w = synth.WORKLOADS[1]
    layer = L.DecoderLayer(w.config_dict(), synth.layer_weights(w), w.dtype, w.positions_needed())
    cache = L.PagedKVCache(layer, w.batch * ((w.positions_needed() + 15) // 16), w.batch)
    x = synth.layer_input(w).cuda()
    xt = synth.decode_input(w, 0).cuda()

    def prefill():
        sids = [cache.add_seq() for _ in range(w.batch)]
        layer.prefill(cache, sids, x)
        return sids

    def prefill_free():
        for s in prefill():
            cache.free_seq(s)

    pre_ms = timed(prefill_free, 50, 5)
    dec_us = []
    for _ in range(10):  # each round: prefill, then the workload's decode steps, timed one by one
        sids = prefill()
        torch.cuda.synchronize()
        for _ in range(w.decode_steps):
            t0 = time.perf_counter()
            layer.decode(cache, sids, xt)
            torch.cuda.synchronize()
            dec_us.append((time.perf_counter() - t0) * 1e6)
        for s in sids:
            cache.free_seq(s)
    cache.close()
    layer.close()
    out[w.name] = {"prefill_ms": round(pre_ms, 4), "decode_us_per_step": round(float(np.median(dec_us)), 1),
                   "batch": w.batch, "seq_len": w.seq_len, "decode_steps": w.decode_steps,
                   "note": "latency of single calls, each synchronised (launch-bound at this size)"}
    log(f"[bench] {w.name}: prefill {pre_ms:.3f} ms, decode step {np.median(dec_us):.1f} us")

    for name in ("llama-7b-layer-prefill", "llama3-70b-layer-prefill"):
        w = synth.PREFILL_JOBS[name]
        log(f"[bench] {name}: generating weights")
        layer = L.DecoderLayer(w.config_dict(), synth.layer_weights(w), "bf16", w.positions_needed())
        cache = L.PagedKVCache(layer, w.batch * ((w.seq_len + 15) // 16), w.batch)
        x = synth.layer_input(w).cuda()
        y = torch.empty((w.batch, w.seq_len, w.hidden_size), dtype=torch.bfloat16, device="cuda")

        def step():
            sids = [cache.add_seq() for _ in range(w.batch)]
            layer.prefill(cache, sids, x, out_dtype="bf16", out=y)
            for s in sids:
                cache.free_seq(s)

        ms = timed(step, min(args.steps, 10), 2)
        fl = sum(prefill_flops(w).values())
        out[name] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.batch * w.seq_len / (ms * 1e-3), 1),
                     "layer_tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                     "layer_mfma_frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "batch": w.batch, "seq_len": w.seq_len}
        log(f"[bench] {name}: {ms:.3f} ms/step")
        cache.close()
        layer.close()
        del x, y
    return out


def run_decode(args, torch, L, synth):
    w = synth.DECODE_JOBS[args.decode_workload]
    log(f"[bench] decode workload {w.name}: weights and cache")
    # positions for the warm-up, timed and profiled steps past the longest context
    max_pos = w.ctx_hi + 2 * args.decode_steps + args.decode_warmup + 1
    model, layers = make_model(args, L, synth, w, max_pos)
    nl = len(layers)
    lens = synth.context_lengths(w)
    nsteps = args.decode_steps
    # room for warm-up, the timed steps and the profiled repeat of them
    nb = int(sum((int(l) + 2 * nsteps + args.decode_warmup + 15) // 16 for l in lens))
    perm = synth.block_permutation(w, nb).tolist()
    cache = make_cache(L, model, layers, nb, w.batch, order=perm)
    sids = []
    for b in range(w.batch):
        sid = cache.add_seq()
        k, v = synth.cache_contents(w, b, int(lens[b]))
        if nl > 1:  # the same contents in every layer's pool
            k, v = k.expand(nl, *k.shape), v.expand(nl, *v.shape)
        cache.write(sid, k.cuda(), v.cuda())
        sids.append(sid)
    xs = [synth.decode_input(w, s).cuda() for s in range(nsteps + args.decode_warmup)]
    out = torch.empty((w.batch, w.hidden_size), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    for s in range(args.decode_warmup):
        model.decode(cache, sids, xs[s], out_dtype="bf16", out=out)
    torch.cuda.synchronize()
    ctx_start = np.array([cache.seq_len(s) for s in sids], dtype=np.int64)
    # timed steps without per-kernel events (at microsecond kernels the event
    # records themselves would show up in the step time) ...
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(nsteps):
        model.decode(cache, sids, xs[args.decode_warmup + s], out_dtype="bf16", out=out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    us = (t1 - t0) * 1e6 / nsteps
    # ... then the same number of steps again with per-kernel HIP events on the
    # layer's stream, for the kernel breakdown (context now longer by nsteps)
    ctx_prof = np.array([cache.seq_len(s) for s in sids], dtype=np.int64)
    profile_all(L, layers, True)
    for s in range(nsteps):
        model.decode(cache, sids, xs[args.decode_warmup + s], out_dtype="bf16", out=out)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    prof = profile_sum(L, layers)
    profile_all(L, layers, False)
    us_prof = (t2 - t1) * 1e6 / nsteps
    G, D = w.num_key_value_heads, w.head_dim
    # keys read per step: every cached key plus the new one, K and V, once per KV group
    keys = float(np.sum(ctx_start + 1)) + w.batch * (nsteps - 1) / 2.0
    kv_bytes = keys * G * D * 2 * 2 * nl
    keys_prof = float(np.sum(ctx_prof + 1)) + w.batch * (nsteps - 1) / 2.0
    kv_bytes_prof = keys_prof * G * D * 2 * 2  # one layer's (one launch of the attention kernel)
    d, I, H = w.hidden_size, w.intermediate_size, w.num_attention_heads
    weight_bytes = 2 * (d * (H + 2 * G) * D + H * D * d + 3 * d * I) * nl
    dom = "attn_decode_split"
    dom_ms = prof[dom][1] / prof[dom][0]
    ach = kv_bytes_prof / (dom_ms * 1e-3) / 1e9
    rec = traffic_record(dom)
    traffic = (round(float(rec["ratio_to_algorithmic"]) * kv_bytes_prof)
               if rec and "ratio_to_algorithmic" in rec else None)
    kern = {n: {"avg_us": round(t / c * 1e3, 2), "launches": c} for n, (c, t) in prof.items()}
    step_bytes = kv_bytes + weight_bytes
    # decode attention plus the norm kernels: their summed event time per
    # step against their algorithmic bytes (K/V once per group, q in, attention
    # out; norm 1 reads x (bf16) and writes its operand; a separate norm 2
    # reads h (fp32) and writes its operand -- at decode sizes that norm runs
    # inside the o_proj GEMM's split-K pass and is not counted here)
    T = w.batch
    an_kernels = [k for k in ("attn_decode_split", "attn_decode_combine", "rms_rowscale", "rms_convert")
                  if k in prof]
    an_us = sum(prof[k][1] / prof[k][0] * 1e3 for k in an_kernels)
    an_bytes = (kv_bytes_prof + 2 * T * H * D * 2                      # K/V, q, attention output
                + (T * d * 2 * 2 if "rms_rowscale" in prof else 0)     # norm 1
                + (T * d * 4 + T * d * 2 if "rms_convert" in prof else 0))  # norm 2
    an_ach = an_bytes / (an_us * 1e-6) / 1e9
    log(f"[bench] decode {us:.1f} us/step ({us_prof:.1f} with per-kernel events), "
        f"{step_bytes / (us * 1e-6) / 1e9:.0f} GB/s whole step")
    res = {
        "workload": w.name, "batch": w.batch, "steps": nsteps, "us_per_step": round(us, 2),
        "us_per_step_profiled": round(us_prof, 2),
        "mean_context": float(np.mean(ctx_start)), "kernels": kern,
        "step_hbm_frac": round(step_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "attn_norms_roofline": {"bound": "hbm", "kernels": an_kernels, "achieved": round(an_ach, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(an_ach / PEAK_HBM_GBS, 4),
                                "bytes_per_step": an_bytes, "us_per_step": round(an_us, 2)},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": kv_bytes_prof, "avg_launch_ms": round(dom_ms, 4)},
    }
    cache.close()
    model.close()
    for layer in layers:
        layer.close()
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, w, n_rows: int):
    """The float64 oracle on the prefill workload, or on a row sample of it (host cores).

    The oracle's work is numpy matmuls; `cores` is the thread count of the BLAS
    pool that runs them (OMP_NUM_THREADS where set), `host_logical_cpus` what
    the host reports."""
    import oracle
    from threadpoolctl import threadpool_info
    ws = synth.layer_weights(w)
    wo = {k: synth.as_f64(v) for k, v in ws.items()}
    x = synth.as_f64(synth.layer_input(w))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    host = {"host_logical_cpus": os.cpu_count(), "cpu_model": cpu_model()}
    if n_rows >= w.seq_len:
        t0 = time.perf_counter()
        oracle.prefill(w.config_dict(), wo, x)
        t = time.perf_counter() - t0
        return {"value": round(w.batch * w.seq_len / t, 2), "unit": "tokens/s", "cores": int(threads),
                "kind": "oracle", **host,
                "sample": f"{w.name}: the whole layer prefill (B {w.batch}, S {w.seq_len}) in float64, {t:.1f} s"}
    rows = np.unique(np.linspace(0, w.seq_len - 1, n_rows).astype(np.int64))
    t0 = time.perf_counter()
    oracle.prefill(w.config_dict(), wo, x, rows=rows[-1:])
    t1 = time.perf_counter()
    oracle.prefill(w.config_dict(), wo, x, rows=rows)
    t2 = time.perf_counter()
    t_kv = t1 - t0                                 # K/V of all tokens + one row
    t_full = t_kv + (t2 - t1 - t_kv) * (w.seq_len / len(rows))
    return {"value": round(w.batch * w.seq_len / t_full, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", **host,
            "sample": (f"{w.name}: K/V of all {w.seq_len} tokens plus outputs of {len(rows)} evenly spaced "
                       f"rows, float64; {t2 - t0:.1f} s measured, full-layer time extrapolated linearly "
                       f"in rows")}


def main():
    from decoder_block_amd import synth
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--decode-warmup", type=int, default=4)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the quick timings of the tiny fp32, LLaMA-7B and LLaMA-3-70B layers")
    ap.add_argument("--cpu-rows", type=int, default=8192, help="oracle rows (>= S: the whole layer)")
    ap.add_argument("--prefill-workload", default="llama3-8b-layer-prefill", choices=sorted(synth.PREFILL_JOBS))
    ap.add_argument("--decode-workload", default="llama3-8b-layer-decode", choices=sorted(synth.DECODE_JOBS))
    ap.add_argument("--stack-layers", type=int, default=1,
                    help="N > 1: time a stack of N layers (own weights) plus the final RMSNorm")
    args = ap.parse_args()
    if args.stack_layers < 1:
        ap.error("--stack-layers must be at least 1")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from decoder_block_amd import llama_layer as L
    L.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    w, pre = run_prefill(args, torch, L, synth)
    dec = None if args.no_decode else run_decode(args, torch, L, synth)
    other = None if args.no_other_workloads else run_other_workloads(args, torch, L, synth)
    cpu = None if args.no_cpu_baseline else cpu_baseline(synth, w, args.cpu_rows)
    line = {
        "metric": METRIC, "value": round(pre["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(pre["ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, random init)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "hidden_size": w.hidden_size,
                   "intermediate_size": w.intermediate_size, "num_attention_heads": w.num_attention_heads,
                   "num_key_value_heads": w.num_key_value_heads, "rope_theta": w.rope_theta,
                   "rms_norm_eps": w.rms_norm_eps,
                   **({"stack_layers": args.stack_layers} if args.stack_layers > 1 else {})},
        "layer_tflops": round(pre["layer_tflops"], 1),
        "layer_mfma_frac": round(pre["layer_tflops"] / PEAK_BF16_TFLOPS, 4),
        "roofline": pre["roofline"],
        "layer_roofline": pre["layer_roofline"],
        "kernels": pre["kernels"],
        "decode": dec,
        "other_workloads": other,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
