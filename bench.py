"""Benchmark: one GPT-2 training step (forward, backward, AdamW) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload gpt2-124m|gpt2-350m]
    python bench.py --workload block-fp32  (one GPT-2 block fwd+bwd in fp32, B=4, T=256)
    python bench.py --workload lmhead-ce   (the tied LM head + CE fwd+bwd alone, N=8192)
    python bench.py --dtype fp16         (the same step in fp16 with dynamic loss scaling)
    python bench.py --decode             (greedy decoding with the KV cache, B=8)
    python bench.py --mlp                (the tiny classifier through the graph autograd)
    python bench.py --probe              (the roofline probes alone: MFMA and HBM rates)
    python bench.py --calibrate-copy     (1 GiB device copies, for HBM counter scaling)

Workload (default): GPT-2 124M — 12 layers, d=768, 12 heads, vocab 50257
(token table padded to 50304 rows), context 1024, batch 8; synthetic seeded
token ids and weights; bf16 MFMA compute with fp32 master weights; AdamW
lr 3e-4, betas (0.9, 0.95), wd 0.1.  Inputs and weights are resident in HBM
before the timed region.  Prints ONE JSON line on stdout (progress on stderr).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "train tokens/sec, GPT-2 124M fwd+bwd+AdamW step at 1 GPU; MFMA util %"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 (MFMA)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

WORKLOADS = {
    "gpt2-124m": dict(L=12, C=768, NH=12, V=50257, V_pad=50304, T=1024, B=8),
    "gpt2-350m": dict(L=24, C=1024, NH=16, V=50257, V_pad=50304, T=1024, B=16),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_flops(L, C, V, T, B, F=None, **_):
    """Algorithmic FLOPs of one training step (forward + backward = 3x forward;
    causal attention counts only the j <= i triangle)."""
    F = 4 * C if F is None else F
    N = B * T
    linear = 2.0 * N * (4 * C * C + 2 * C * F)        # qkv, proj, fc, fcproj
    attn = 2.0 * B * C * T * (T + 1)                   # QK^T and PV, causal
    head = 2.0 * N * C * V
    return 3.0 * (L * (linear + attn) + head)


def cpu_baseline(w, dtype="bf16"):
    """Time the CPU oracle (float64 NumPy, as it stands) on a bounded sample of
    the same workload: one training step of the same model on one sequence of
    a reduced length, scaled to tokens/s."""
    import numpy as np
    import oracle  # noqa: F401  (test infrastructure: the baseline leg only)
    from oracle import gpt2 as og
    from autograd_transformer_amd import synthetic as syn
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OPENBLAS_NUM_THREADS", str(cores))
    shape = syn.ModelShape(w["L"], w["C"], w["NH"], w["V"], w["T"])
    cfg = og.GPTConfig(n_layer=w["L"], n_embd=w["C"], n_head=w["NH"], vocab=w["V"],
                       block_size=w["T"])
    p = {k: v.astype(np.float64) for k, v in syn.gpt2_params(shape, seed=3).items()}
    zeros = {k: np.zeros_like(v) for k, v in p.items()}
    T = w["T"]
    tok, tgt = syn.gpt2_tokens(1, T, w["V"], seed=3)
    t0 = time.perf_counter()
    if dtype == "fp16":
        og.train_step_scaled(p, zeros, dict(zeros), 1, tok, tgt, cfg, 65536.0, 0)
    else:
        og.train_step(p, zeros, dict(zeros), 1, tok, tgt, cfg, "bf16")
    dt = time.perf_counter() - t0
    return {"value": round(T / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one full {w['L']}-layer training step (fwd+bwd+AdamW, {dtype} storage "
                      f"rounding, float64 NumPy) on 1 sequence of {T} tokens; {dt:.1f} s"}


def _counter_record(key, what, kernel, field):
    """`field` of `kernel` in the committed rocprofv3 counter summary
    profiles/<key>_<what>.json, or None when there is none or the library
    sources changed since the counters were taken."""
    from autograd_transformer_amd.pmc_traffic import source_digest
    path = os.path.join(ROOT, "profiles", f"{key}_{what}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_digest") != source_digest():
        log(f"[bench] {os.path.basename(path)} was measured on other sources: {field} null")
        return None
    k = rec["kernels"].get(kernel)
    if k is not None:
        return k[field]
    # A timer name can stand for several template instances that rocprofv3
    # lists apart ("gemm_kernel<f32>" covers every fp32 layout and tile):
    # combine them, bytes weighted by launches, utilisation by busy time.
    base, _, targ = kernel.partition("<")
    dtype = {"f32>": "float", "bf16>": "__bf16"}.get(targ)
    hits = [v for n, v in rec["kernels"].items()
            if n.split("<")[0] == base and
            (dtype is None or n.partition("<")[2].split(",")[0].strip(" >") == dtype)]
    if not hits:
        return None
    wkey = "gui_active" if field == "mfma_busy" else "launches"
    w = sum(v[wkey] for v in hits)
    if w <= 0:
        return None
    val = sum(v[field] * v[wkey] for v in hits) / w
    return round(val, 4) if field == "mfma_busy" else int(round(val))


def counter_fields(roof, key):
    """roofline.traffic (HBM bytes per launch of the dominant kernel, from
    FETCH_SIZE / WRITE_SIZE scaled by a device copy) and roofline.mfma_busy
    (its MFMA utilisation from SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE),
    both from the committed counter summaries of workload `key`."""
    roof["traffic"] = _counter_record(key, "hbm_traffic", roof["kernel"], "hbm_bytes_per_launch")
    roof["mfma_busy"] = _counter_record(key, "mfma_busy", roof["kernel"], "mfma_busy")


def bound_of(k, peak_mfma=PEAK_BF16_TFLOPS):
    """The roofline that bounds a kernel: MFMA when its algorithmic intensity
    (FLOPs per HBM byte) reaches the ridge point of the two peaks, else HBM."""
    if k["flops"] > 0 and (k["bytes"] <= 0 or
                           k["flops"] / k["bytes"] >= peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)):
        return "mfma"
    return "hbm"


def roofline(kernels, steps, ms, peak_mfma=PEAK_BF16_TFLOPS):
    """Roofline of the dominant kernel (largest total time in the profiled
    pass): algorithmic FLOPs or bytes per launch over its average launch."""
    dom = max(kernels, key=lambda k: k["ms"])
    avg_ms = dom["ms"] / dom["calls"]
    if bound_of(dom, peak_mfma) == "mfma":
        achieved = dom["flops"] / dom["calls"] / (avg_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_mfma,
                "unit": "TFLOP/s"}
    else:
        achieved = dom["bytes"] / dom["calls"] / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(achieved / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = dom["name"]
    roof["calls_per_step"] = dom["calls"] / steps
    roof["avg_launch_us"] = round(avg_ms * 1e3, 2)
    roof["share_of_step"] = round(dom["ms"] / steps / ms, 4)
    return roof


def measured_peaks(ctx):
    """The roofline probes run live: dense bf16 MFMA on register operands
    (the best of 2 and 4 waves per SIMD, 16 and 32 accumulators) and a
    streaming HBM read and copy over 4 GiB."""
    import torch
    import autograd_transformer_amd as tt
    mfma = max(tt.tt_probe_mfma(ctx, w, a, 4000) for w, a in ((2, 32), (4, 16), (4, 32)))
    buf = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    read = tt.tt_probe_hbm(ctx, buf, copy=False)
    copy = tt.tt_probe_hbm(ctx, buf, copy=True)
    del buf
    return {"mfma_bf16_tflops": round(mfma, 1), "hbm_read_gbs": round(read, 1),
            "hbm_copy_gbs": round(copy, 1)}


def add_measured(roof, peaks):
    """The dominant kernel's rate against the live probe's ceiling too."""
    if peaks is None:
        return
    if roof["bound"] == "mfma" and roof["peak"] == PEAK_BF16_TFLOPS:
        m = peaks["mfma_bf16_tflops"]
    elif roof["bound"] == "hbm":
        m = peaks["hbm_copy_gbs"]
    else:
        return
    roof["peak_measured"] = m
    roof["frac_of_measured"] = round(roof["achieved"] / m, 4)


def hbm_kernels(kernels, steps, ms, key, min_share=0.005):
    """The HBM-bound kernels of the profiled pass (below the ridge point) with
    at least `min_share` of the step: algorithmic bytes per launch over the
    average launch, against 8 TB/s, and (while the committed counter summary
    matches the sources) the same with the bytes rocprofv3 counted."""
    rows = []
    for k in sorted(kernels, key=lambda k: -k["ms"]):
        if k["bytes"] <= 0 or bound_of(k) != "hbm" or k["ms"] / steps < min_share * ms:
            continue
        avg_s = k["ms"] / k["calls"] / 1e3
        gbs = k["bytes"] / k["calls"] / avg_s / 1e9
        row = {"kernel": k["name"], "ms_per_step": round(k["ms"] / steps, 4),
               "achieved_gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
        counted = _counter_record(key, "hbm_traffic", k["name"], "hbm_bytes_per_launch")
        row["counter_gbs"] = None if counted is None else round(counted / avg_s / 1e9, 1)
        rows.append(row)
    return rows


def log_kernels(kernels, steps, n=8):
    for k in sorted(kernels, key=lambda k: -k["ms"])[:n]:
        rate = (f"{k['flops'] / (k['ms'] / 1e3) / 1e12:7.1f} TFLOP/s" if bound_of(k) == "mfma" else
                f"{k['bytes'] / (k['ms'] / 1e3) / 1e9:7.1f} GB/s")
        log(f"[bench]   {k['ms'] / steps:7.3f} ms/step  {k['calls'] // steps:4d} calls  "
            f"{rate}  {k['name']}")


def cpu_decode_baseline(w, P):
    """The oracle's greedy step as it stands (the whole sequence recomputed, no
    cache), one sequence at context P, scaled to tokens/s."""
    import numpy as np
    import oracle  # noqa: F401  (test infrastructure: the baseline leg only)
    from oracle import gpt2 as og
    from autograd_transformer_amd import synthetic as syn
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OPENBLAS_NUM_THREADS", str(cores))
    shape = syn.ModelShape(w["L"], w["C"], w["NH"], w["V"], w["T"])
    cfg = og.GPTConfig(n_layer=w["L"], n_embd=w["C"], n_head=w["NH"], vocab=w["V"],
                       block_size=w["T"])
    p = {k: v.astype(np.float64) for k, v in syn.gpt2_params(shape, seed=3).items()}
    tok, _ = syn.gpt2_tokens(1, P, w["V"], seed=5)
    t0 = time.perf_counter()
    og.greedy_generate(p, tok, 1, cfg, "bf16")
    dt = time.perf_counter() - t0
    return {"value": round(1.0 / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one greedy step of one sequence at context {P} (full forward recomputed, "
                      f"float64 NumPy, bf16 storage rounding); {dt:.1f} s"}


def decode_main(args, w):
    """Greedy decoding with the KV cache: prefill P tokens per sequence, then
    time single-token decode steps (logits, argmax) at growing positions."""
    import torch
    import autograd_transformer_amd as tt
    from autograd_transformer_amd import synthetic as syn
    L, C, NH, V, V_pad, T, B = (w[k] for k in ("L", "C", "NH", "V", "V_pad", "T", "B"))
    P = T // 2
    K = min(args.steps, (T - P - args.warmup) // 2)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    ctx = tt.Context(arena_bytes=(64 << 30) if L > 12 else (24 << 30), stream=stream)
    model = tt.Model(ctx, L=L, C=C, NH=NH, V=V, T_max=T, B_max=B, mode="bf16", V_pad=V_pad)
    model.load(syn.gpt2_params(syn.ModelShape(L, C, NH, V, T), seed=3))
    cache = tt.KVCache(ctx, model, B)
    prompt, _ = syn.gpt2_tokens(B, P, V, seed=5)
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    tt.tt_model_prefill(ctx, model, cache, B, P, torch.from_numpy(prompt).cuda(), None, nxt)
    cur = torch.zeros(B, dtype=torch.int32, device="cuda")
    pos = P

    def step():
        nonlocal pos
        cur.copy_(nxt)
        tt.tt_model_decode(ctx, model, cache, B, pos, cur, None, nxt)
        pos += 1

    for _ in range(args.warmup):
        step()
    ctx.sync()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0 = pos
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    ctx.profile(True)
    for _ in range(K):
        step()
    kernels = ctx.profile_report()
    ctx.profile(False)
    ctx.sync()
    value = B / (ms / 1e3)
    log(f"[bench] decode: {ms * 1e3:.1f} us/step  {value:,.0f} tokens/s  (B={B}, positions "
        f"{p0}..{p0 + K - 1})")
    out = {
        "metric": "greedy decode tokens/sec with KV cache, GPT-2 124M at 1 GPU",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded uniform token ids, N(0,0.02) weights)",
        "config": {"workload": f"{args.workload} greedy decode, KV cache, bf16", "batch": B,
                   "prompt": P, "positions": [p0, p0 + K - 1], "parallelism": "single GPU"},
        "roofline": roofline(kernels, K, ms),
    }
    log_kernels(kernels, K)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle's greedy step ...")
        out["cpu_baseline"] = cpu_decode_baseline(w, P)
    cache.close()
    model.close()
    ctx.close()
    print(json.dumps(out), flush=True)


def mlp_main(args):
    """The tiny classifier (x [64,3] -> Linear 3->32 -> GELU -> Linear 32->4 ->
    mean cross-entropy -> SGD lr 0.1) recorded as a tt_graph: per-step time of
    the eager walk and of the step captured as one HIP graph."""
    import torch
    import autograd_transformer_amd as tt
    from autograd_transformer_amd import synthetic as syn
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    ctx = tt.Context(arena_bytes=1 << 26, stream=stream)
    d = syn.mlp_inputs(seed=1)
    P = {k: torch.from_numpy(d[k]).float().cuda() for k in ("W1", "b1", "W2", "b2")}
    G = {k: torch.zeros_like(v) for k, v in P.items()}
    g = tt.Graph(ctx)
    x = g.leaf(torch.from_numpy(d["x"]).float().cuda())
    ids = {k: g.leaf(P[k], G[k]) for k in P}
    h = g.gelu(g.add(g.matmul(x, ids["W1"]), ids["b1"]))
    loss = g.cross_entropy(g.add(g.matmul(h, ids["W2"]), ids["b2"]),
                           torch.from_numpy(d["labels"]).int().cuda())

    def eager():
        g.forward(loss)
        g.zero_grad()
        g.backward(loss)
        for k in P:
            tt.tt_sgd_step(ctx, P[k], G[k], 0.1)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    K = max(args.steps, 200)
    for _ in range(args.warmup):
        eager()
    us_eager = timed(eager, K)
    ctx.profile(True)
    for _ in range(K):
        eager()
    kernels = ctx.profile_report()
    ctx.profile(False)
    launches = sum(k["calls"] for k in kernels) / K
    g.capture_sgd_step(loss, 0.1)
    for _ in range(args.warmup):
        g.step()
    us_graph = timed(g.step, K)
    final = float(g.value(loss).item())
    # the same step as one kernel (everything in one workgroup's LDS)
    Pf = {k: torch.from_numpy(d[k]).float().cuda() for k in P}
    xf = torch.from_numpy(d["x"]).float().cuda()
    yf = torch.from_numpy(d["labels"]).int().cuda()
    lf = torch.zeros(1, device="cuda")

    def fused():
        tt.tt_mlp_step(ctx, xf, yf, Pf["W1"], Pf["b1"], Pf["W2"], Pf["b2"], 0.1, lf)

    for _ in range(args.warmup):
        fused()
    us_fused = timed(fused, K)
    ctx.profile(True)
    for _ in range(K):
        fused()
    fk = ctx.profile_report()
    ctx.profile(False)
    log(f"[bench] tiny classifier: graph eager {us_eager:.1f} us/step ({launches:.0f} launches), "
        f"graph captured {us_graph:.1f} us/step, one kernel {us_fused:.1f} us/step, "
        f"loss {final:.4f}")
    out = {
        "metric": "tiny-classifier SGD step time (x[64,3], Linear 3->32, GELU, Linear 32->4, "
                  "mean CE, SGD lr 0.1)",
        "value": round(us_fused, 2), "unit": "us/step", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(us_fused / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,1) inputs and weights, uniform labels)",
        "config": {"workload": "tiny classifier step, 64 samples, one fused kernel",
                   "graph_eager_us_per_step": round(us_eager, 2),
                   "graph_launches_per_step": launches,
                   "graph_captured_us_per_step": round(us_graph, 2),
                   "parallelism": "single GPU"},
        # one workgroup of float32 vector arithmetic: launch-latency bound at
        # this size (the roofline figure is for the record, not a target)
        "roofline": roofline(fk, K, us_fused / 1e3, peak_mfma=157.3),
    }
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle import gpt2 as og  # test infrastructure: the baseline leg only
        W = {k: d[k].astype(np.float64) for k in P}
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 2.0:
            og.mlp_step(d["x"], W["W1"], W["b1"], W["W2"], W["b2"], d["labels"])
            n += 1
        dt = (time.perf_counter() - t0) / n
        out["cpu_baseline"] = {"value": round(dt * 1e6, 2), "unit": "us/step", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} oracle steps of the same classifier (float64 "
                                         f"NumPy) in {n * dt:.1f} s"}
    g.close()
    ctx.close()
    print(json.dumps(out), flush=True)


def timed_steps(step, stream, warmup, steps):
    """Warm-up, then `steps` steps with a HIP event on `stream` after each
    (the first and last bracket them all): ms/step over the whole run, and
    the sorted per-step times."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[-1]) / steps, per_step


def profiled(ctx, step, steps):
    ctx.profile(True)
    for _ in range(steps):
        step()
    kernels = ctx.profile_report()
    ctx.profile(False)
    ctx.sync()
    return kernels


def oracle_rate(fn, min_s=10.0):
    """Run fn repeatedly for about min_s seconds; seconds per call, calls."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            return dt / n, n


def block_main(args):
    """One pre-LN GPT-2 block, forward and backward, in fp32 through
    tt_block_fwd / tt_block_bwd: B=4, T=256, C=768, 12 heads, MLP 3072;
    x ~ N(0,1), weights ~ N(0,0.02), LN 1/0, biases 0, upstream grad ~ N(0,1)
    (weight gradients accumulate, as the call defines)."""
    import numpy as np
    import torch
    import autograd_transformer_amd as tt
    from autograd_transformer_amd import synthetic as syn
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    d = syn.block_inputs(seed=2)
    B, T, C, NH, F = d["B"], d["T"], d["C"], d["n_head"], d["F"]
    ctx = tt.Context(arena_bytes=4 << 30, stream=stream)
    w = {k: torch.from_numpy(v).cuda() for k, v in d["w"].items()}
    g = {k: torch.zeros_like(v) for k, v in w.items()}
    x, dy = torch.from_numpy(d["x"]).cuda(), torch.from_numpy(d["dy"]).cuda()
    y, dx = torch.empty_like(x), torch.empty_like(x)
    saved = tt.BlockSaved(ctx, B, T, C, NH, F, "f32")

    def step():
        tt.tt_block_fwd(ctx, saved, w, x, y)
        tt.tt_block_bwd(ctx, saved, w, dy, dx, g)

    K = max(args.steps, 50)
    ms, per_step = timed_steps(step, stream, args.warmup, K)
    kernels = profiled(ctx, step, K)
    flops = step_flops(L=1, C=C, V=0, T=T, B=B, F=F)
    tflops = flops / (ms / 1e3) / 1e12
    log(f"[bench] block fp32: {ms * 1e3:.1f} us/step  {tflops:.1f} TFLOP/s "
        f"({flops / 1e9:.2f} GFLOP)")
    out = {
        "metric": "single GPT-2 block fwd+bwd time, fp32 (B=4, T=256, d=768, 12 heads, MLP 3072)",
        "value": round(ms * 1e3, 2), "unit": "us/step", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "ms_median": round(per_step[K // 2], 5), "ms_min": round(per_step[0], 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,1) input and upstream gradient, N(0,0.02) weights)",
        "config": {"workload": "single GPT-2 block fwd+bwd, fp32, B=4 T=256 C=768 NH=12 F=3072",
                   "tokens": B * T, "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "roofline": roofline(kernels, K, ms, peak_mfma=PEAK_FP32_TFLOPS),
    }
    counter_fields(out["roofline"], "block-fp32_b4_t256")
    out["hbm_kernels"] = hbm_kernels(kernels, K, ms, "block-fp32_b4_t256")
    log_kernels(kernels, K)
    if not args.no_cpu_baseline:
        from oracle import gpt2 as og  # test infrastructure: the baseline leg only
        cores = len(os.sched_getaffinity(0))
        w64 = {k: v.astype(np.float64) for k, v in d["w"].items()}

        def ref():
            _, cache = og.block_fwd(d["x"], w64, NH, "f32")
            og.block_bwd(cache, w64, d["dy"], NH, "f32")
        dt, n = oracle_rate(ref)
        out["cpu_baseline"] = {"value": round(dt * 1e6, 1), "unit": "us/step", "cores": cores,
                               "kind": "oracle",
                               "sample": f"{n} full block fwd+bwd steps of the same workload "
                                         f"(float64 NumPy) in {n * dt:.1f} s"}
    saved.close()
    ctx.close()
    print(json.dumps(out), flush=True)


def lmhead_main(args):
    """The tied LM head + mean cross-entropy, forward and backward, alone
    (tt_lmhead_ce_fwdbwd): hidden [8192, 768] bf16 ~ N(0,1), W_emb [50257, 768]
    bf16 ~ N(0,0.02), targets uniform; logits, loss, dHidden and dW_emb with
    float32 accumulation."""
    import numpy as np
    import torch
    import autograd_transformer_amd as tt
    from autograd_transformer_amd import synthetic as syn
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    N, C, V = 8192, 768, 50257
    d = syn.lmhead_inputs(seed=4, N=N, C=C, V=V)
    ctx = tt.Context(arena_bytes=4 << 30, stream=stream)
    h = torch.from_numpy(d["h"]).to(torch.bfloat16).cuda()
    wte = torch.from_numpy(d["wte"]).to(torch.bfloat16).cuda()
    tgt = torch.from_numpy(d["targets"]).cuda()
    loss = torch.zeros(1, device="cuda")
    dh = torch.empty(N, C, device="cuda")
    dwte = torch.zeros(V, C, device="cuda")

    def step():
        tt.tt_lmhead_ce_fwdbwd(ctx, "bf16", N, C, V, h, wte, tgt, loss, dh, dwte)

    K = args.steps
    ms, per_step = timed_steps(step, stream, args.warmup, K)
    kernels = profiled(ctx, step, K)
    flops = 3 * 2.0 * N * C * V
    tflops = flops / (ms / 1e3) / 1e12
    value = N / (ms / 1e3)
    log(f"[bench] LM head + CE: {ms:.3f} ms/step  {value:,.0f} tokens/s  {tflops:.1f} TFLOP/s")
    out = {
        "metric": "fused LM head + cross-entropy fwd+bwd tokens/sec (hidden [8192,768] x "
                  "W_emb [50257,768], bf16, fp32 accumulation)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "ms_median": round(per_step[K // 2], 5), "ms_min": round(per_step[0], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden, N(0,0.02) W_emb, uniform targets)",
        "config": {"workload": "LM head + CE fwd+bwd, N=8192 C=768 V=50257, bf16 / fp32 acc",
                   "tokens": N, "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline(kernels, K, ms),
    }
    counter_fields(out["roofline"], "lmhead-ce_n8192_v50257")
    out["hbm_kernels"] = hbm_kernels(kernels, K, ms, "lmhead-ce_n8192_v50257")
    add_measured(out["roofline"], measured_peaks(ctx))
    log_kernels(kernels, K)
    if not args.no_cpu_baseline:
        from oracle import ops as oo  # test infrastructure: the baseline leg only
        cores = len(os.sched_getaffinity(0))
        os.environ.setdefault("OPENBLAS_NUM_THREADS", str(cores))
        rows = 512
        h64 = d["h"][:rows].astype(np.float64)
        w64 = d["wte"].astype(np.float64)

        def ref():
            oo.lmhead_ce_fwdbwd(h64, w64, d["targets"][:rows])
        dt, n = oracle_rate(ref)
        out["cpu_baseline"] = {"value": round(rows / dt, 2), "unit": "tokens/s", "cores": cores,
                               "kind": "oracle",
                               "sample": f"{n} oracle LM head + CE fwd+bwd calls on the first "
                                         f"{rows} of the 8192 rows (float64 NumPy) in "
                                         f"{n * dt:.1f} s"}
    ctx.close()
    print(json.dumps(out), flush=True)


def probe_main(args):
    """The roofline probes alone, several shapes of each."""
    import torch
    import autograd_transformer_amd as tt
    torch.cuda.set_device(0)
    ctx = tt.Context(arena_bytes=1 << 28)
    res = {}
    for w in (1, 2, 4):
        for a in (8, 16, 32):
            res[f"mfma_bf16_w{w}_acc{a}"] = round(tt.tt_probe_mfma(ctx, w, a, 8000), 1)
    buf = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    res["hbm_read_gbs"] = round(tt.tt_probe_hbm(ctx, buf, copy=False), 1)
    res["hbm_copy_gbs"] = round(tt.tt_probe_hbm(ctx, buf, copy=True), 1)
    # per-CU ceilings in shader clocks
    cu = {}
    cu["lds_read_bytes_per_clk"] = round(tt.tt_probe_lds(ctx, mfma=False)[0], 1)
    b, t = tt.tt_probe_lds(ctx, mfma=True)
    cu["lds_read_feeding_mfma_bytes_per_clk"] = round(b, 1)
    cu["lds_read_feeding_mfma_tflops"] = round(t, 1)
    src = buf[: (1 << 29) // 4]   # 512 MiB of the probe buffer
    cu["lds_load_l2_bytes_per_clk"] = round(tt.tt_probe_lds_load(ctx, src, resident=True), 1)
    cu["lds_load_hbm_bytes_per_clk"] = round(tt.tt_probe_lds_load(ctx, src, resident=False), 1)
    for i, name in enumerate(tt.ISSUE_PROBES):
        cu[f"clk_per_instr_{name}"] = [round(v, 2) for v in tt.tt_probe_issue(ctx, i)]
    res["per_cu"] = cu
    ctx.close()
    print(json.dumps({"probe": "roofline", "peak_vendor": {"mfma_bf16_tflops": PEAK_BF16_TFLOPS,
                                                           "hbm_gbs": PEAK_HBM_GBS},
                      "measured": res}), flush=True)


def step_products(L, C, NH, V, V_pad, T, B, F=None):
    """Every matrix product of one training step as (M, N, K, count, layout):
    'nt' = A [M,K] times B given as [N,K] (both reduced along their rows:
    the forward and activation-gradient products), 'tn' = A given as [K,M]
    times B [K,N] (both token-major: the weight gradients)."""
    F = F or 4 * C
    M = B * T
    per_layer = [(M, 3 * C, C, "nt"), (M, C, C, "nt"), (M, F, C, "nt"), (M, C, F, "nt"),   # forward
                 (M, F, C, "nt"), (M, C, F, "nt"), (M, C, C, "nt"), (M, C, 3 * C, "nt"),   # dX
                 (C, 3 * C, M, "tn"), (C, C, M, "tn"), (C, F, M, "tn"), (F, C, M, "tn")]   # dW
    out = [(m, n, k, L, lay) for m, n, k, lay in per_layer]
    out += [(M, V_pad, C, 1, "nt"), (M, C, V_pad, 1, "nt"), (V_pad, C, M, 1, "tn")]  # LM head
    return out


def vendor_main(args, w):
    """The vendor library on the step's products, for scale: hipBLASLt
    (through torch.matmul; bf16 in and out, no epilogues) on every product of
    the training step, summed per step, next to this library's GEMM kernels
    in the same step (the profiled pass's kernels named gemm*, with their
    fused bias / GELU / residual / column-sum epilogues)."""
    import torch
    import autograd_transformer_amd as tt
    from autograd_transformer_amd import synthetic as syn
    L, C, NH, V, V_pad, T, B = (w[k] for k in ("L", "C", "NH", "V", "V_pad", "T", "B"))
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    params = syn.gpt2_params(syn.ModelShape(L, C, NH, V, T), seed=3)
    tok, tgt = syn.gpt2_tokens(B, T, V, seed=3)
    ctx = tt.Context(arena_bytes=64 << 30 if L > 12 else 24 << 30, stream=stream)
    model = tt.Model(ctx, L=L, C=C, NH=NH, V=V, T_max=T, B_max=B, mode="bf16", V_pad=V_pad)
    model.load(params)
    del params
    tok_d, tgt_d = torch.from_numpy(tok).cuda(), torch.from_numpy(tgt).cuda()
    loss = torch.zeros(1, device="cuda")
    t = 1
    for _ in range(args.warmup):
        tt.tt_train_step(ctx, model, B, T, tok_d, tgt_d, 3e-4, 0.9, 0.95, 1e-8, 0.1, t, loss)
        t += 1
    ctx.sync()
    ctx.profile(True)
    for _ in range(args.steps):
        tt.tt_train_step(ctx, model, B, T, tok_d, tgt_d, 3e-4, 0.9, 0.95, 1e-8, 0.1, t, loss)
        t += 1
    kernels = ctx.profile_report()
    ctx.profile(False)
    ctx.sync()
    ours = sum(k["ms"] for k in kernels if k["name"].startswith("gemm")) / args.steps
    ours_flops = sum(k["flops"] for k in kernels if k["name"].startswith("gemm")) / args.steps
    model.close()
    ctx.close()
    rows, total = [], 0.0
    for m, n, k, count, lay in step_products(L, C, NH, V, V_pad, T, B):
        if lay == "nt":
            a = torch.randn(m, k, device="cuda").to(torch.bfloat16)
            b = torch.randn(n, k, device="cuda").to(torch.bfloat16)
            run = lambda: a @ b.t()
        else:
            a = torch.randn(k, m, device="cuda").to(torch.bfloat16)
            b = torch.randn(k, n, device="cuda").to(torch.bfloat16)
            run = lambda: a.t() @ b
        for _ in range(3):
            run()
        reps = 20 if m * n * k < 2e10 else 5
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        total += ms * count
        rows.append({"M": m, "N": n, "K": k, "per_step": count, "layout": lay,
                     "us": round(ms * 1e3, 1), "tflops": round(2.0 * m * n * k / ms / 1e9, 1)})
        del a, b
    print(json.dumps({"comparison": "vendor GEMM library on the step's products",
                      "workload": f"{args.workload} B={B} T={T}",
                      "ours_gemm_ms_per_step": round(ours, 3),
                      "ours_gemm_tflops": round(ours_flops / ours / 1e9, 1),
                      "vendor_gemm_ms_per_step": round(total, 3),
                      "vendor_gemm_tflops": round(ours_flops / total / 1e9, 1),
                      "products": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2-124m",
                    choices=sorted(WORKLOADS) + ["block-fp32", "lmhead-ce"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16"],
                    help="16-bit format of the training step (fp16: dynamic loss scaling)")
    ap.add_argument("--decode", action="store_true",
                    help="measure greedy decoding with the KV cache instead of training")
    ap.add_argument("--mlp", action="store_true",
                    help="measure the tiny classifier's step through the graph autograd")
    ap.add_argument("--probe", action="store_true",
                    help="only run the roofline probes (MFMA and HBM) and exit")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the vendor GEMM library (torch.matmul) on the step's products "
                         "next to this library's GEMM kernels, and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 5 device copies of 1 GiB (reference for rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE scaling) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the data-parallel sharding is described in the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.calibrate_copy:
        from autograd_transformer_amd.pmc_traffic import COPY_BYTES
        src = torch.ones(COPY_BYTES // 4, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": COPY_BYTES,
                          "bytes_written": COPY_BYTES, "launches": 5}), flush=True)
        return
    import autograd_transformer_amd as tt
    from autograd_transformer_amd import synthetic as syn

    if args.mlp:
        mlp_main(args)
        return
    if args.probe:
        probe_main(args)
        return
    if args.workload == "block-fp32":
        block_main(args)
        return
    if args.workload == "lmhead-ce":
        lmhead_main(args)
        return
    w = WORKLOADS[args.workload]
    if args.vendor_gemm:
        vendor_main(args, w)
        return
    if args.decode:
        decode_main(args, w)
        return
    L, C, NH, V, V_pad, T, B = (w[k] for k in ("L", "C", "NH", "V", "V_pad", "T", "B"))
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    log(f"[bench] {args.workload}: generating synthetic weights ...")
    shape = syn.ModelShape(L, C, NH, V, T)
    params = syn.gpt2_params(shape, seed=3)
    tok, tgt = syn.gpt2_tokens(B, T, V, seed=3)
    arena = 64 << 30 if L > 12 else 24 << 30
    ctx = tt.Context(arena_bytes=arena, stream=stream)
    model = tt.Model(ctx, L=L, C=C, NH=NH, V=V, T_max=T, B_max=B, mode=args.dtype, V_pad=V_pad)
    model.load(params)
    del params
    tok_d = torch.from_numpy(tok).cuda()
    tgt_d = torch.from_numpy(tgt).cuda()
    loss = torch.zeros(1, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.95, 1e-8, 0.1

    def step(t):
        tt.tt_train_step(ctx, model, B, T, tok_d, tgt_d, lr, b1, b2, eps, wd, t, loss, flag)

    log(f"[bench] warmup {args.warmup} steps")
    t = 1
    for _ in range(args.warmup):
        step(t)
        t += 1
    ctx.sync()
    log(f"[bench] timing {args.steps} steps")
    # an event after every step: the first and last bracket the K steps, the
    # ones between give each step's own time (median, min)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(t)
        t += 1
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ctx.sync()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    last_loss = float(loss.item())
    if not math.isfinite(last_loss) or int(flag.item()) != 0:
        log(f"[bench] WARNING: non-finite loss {last_loss} or a dropped (overflowed) step")
    # Second pass over the same number of steps with every kernel launch
    # bracketed by HIP events on the context stream: per-kernel durations for
    # the roofline of the dominant kernel (events add small gaps between
    # kernels, so this pass is not the throughput figure).
    ctx.profile(True)
    for _ in range(args.steps):
        step(t)
        t += 1
    kernels = ctx.profile_report()
    ctx.profile(False)
    ctx.sync()
    tokens = B * T
    flops = step_flops(**w)
    value = tokens / (ms / 1e3)
    tflops = flops / (ms / 1e3) / 1e12
    log(f"[bench] {ms:.3f} ms/step  {value:,.0f} tokens/s  {tflops:.1f} TFLOP/s "
        f"(wall {wall:.2f}s)  loss {last_loss:.4f}")

    out = {
        "metric": METRIC if args.workload == "gpt2-124m" else METRIC.replace("GPT-2 124M", "GPT-2 350M"),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_median": round(per_step[len(per_step) // 2], 4),
        "ms_min": round(per_step[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded uniform token ids, N(0,0.02) weights)",
        "config": {"workload": f"{args.workload} train step (fwd+bwd+AdamW), {args.dtype} MFMA / "
                               f"fp32 master" + (", dynamic loss scaling" if args.dtype == "fp16"
                                                 else ""),
                   "global_batch": B, "seq_len": T, "layers": L, "d_model": C, "heads": NH,
                   "vocab": V, "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "loss": round(last_loss, 5),
    }
    out["roofline"] = roofline(kernels, args.steps, ms)
    ckey = f"{args.workload}_b{B}_t{T}" + ("" if args.dtype == "bf16" else "_" + args.dtype)
    counter_fields(out["roofline"], ckey)
    out["hbm_kernels"] = hbm_kernels(kernels, args.steps, ms, ckey)
    # the live probes, after the timed and profiled passes
    add_measured(out["roofline"], measured_peaks(ctx))
    log_kernels(kernels, args.steps)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(w, args.dtype)
    model.close()
    ctx.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
