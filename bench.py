"""Benchmark of the layer-streamed training step on one MI355X.

Workload (default): Qwen2.5-7B-shaped decoder, random N(0, 0.02^2) init,
batch 16 x seq 1024 uniform random token ids (a fresh seeded batch every
step), checkpoint interval 4; bf16 weights stream from pinned host memory,
fp32 master + Adam states on the host, CPU Adam, weight loads up to 3 layers
ahead of compute.  Layers 1-8 (at most a third of the layers) stay on the
device between steps: each one's updated copy streams in during the
backward right after its host update (--resident-layers).  A step is one
full mt_stream_step (forward, head, segment re-forward, backward, gradient
offload, CPU Adam of every unit).

Prints one JSON line: sustained TFLOPS by the 6ND + 12LHT^2 formula
(MegaTrain listing page, Table 7 caption; T^2 term not scaled by the batch)
plus tokens/s, the roofline of the dominant kernel (the GEMM instantiation
or attention kernel with the largest total time in the step, every launch
timed with HIP events on the compute stream inside the timed steps), the
same steps under the pages' own schedule (every layer streamed every step,
double buffering, per-layer recompute in the backward), and the CPU oracle
timed on a bounded sample.  --ablation adds the listing page's Table 4
ablation (prefetch depth, slab pool, checkpoint interval) on the same model.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (no sparsity)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_hbm_traffic_qwen2.5-7b-b16-t1024.md")


def gemm_sources_sha256():
    import hashlib
    src = os.path.join(ROOT, "layer_streamed_amd", "csrc")
    return hashlib.sha256(open(os.path.join(src, "gemm.hip"), "rb").read()
                          + open(os.path.join(src, "common.h"), "rb").read()).hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None if the summary covers another kernel or the GEMM sources changed
    since the counters were taken."""
    import re
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    name = re.search(r"^kernel: (.+)$", text, re.M)
    sha = re.search(r"source_sha256: ([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    if not (name and sha and val) or name.group(1).strip() != kernel:
        return None
    if sha.group(1) != gemm_sources_sha256():
        return None
    return int(val.group(1))


def init_weights(model, shape, seed):
    """N(0, 0.02^2) matrices drawn on the GPU (plumbing only), gains 1."""
    import numpy as np
    import torch

    import synth
    g = torch.Generator(device="cuda").manual_seed(seed)
    shapes = synth.param_shapes(shape)
    for name in synth.param_names(shape):
        shp = shapes[name]
        if name.endswith("norm"):
            model.set_param(name, np.ones(shp, np.float32))
            continue
        t = torch.randn(shp, device="cuda", generator=g, dtype=torch.float32).mul_(0.02)
        model.set_param(name, t.cpu().numpy())
        del t


def cpu_baseline(shape):
    """The oracle on a bounded sample of the same workload: one decoder layer
    at the real width on a few sequences (forward, the re-forward share,
    recompute and backward), the head on the same sequences, and Adam over
    one layer's parameters (about 10-15 s of CPU work); extrapolated to the
    full step."""
    import numpy as np

    import synth
    from oracle import decoder as D
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=os.cpu_count())
    except Exception:
        cores = os.cpu_count()
    T = min(shape.seq, 1024)
    nb = max(1, min(4, shape.batch * shape.seq // T))  # sequences in the sample
    s1 = shape.with_(batch=nb, seq=T)
    w = synth.make_weights(s1, seed=0, names=synth.layer_param_names(0))
    w = {k.split(".")[-1]: v for k, v in w.items()}
    rng = np.random.default_rng(0)
    x = rng.standard_normal((nb, T, shape.hidden)).astype(np.float32)
    dy = (rng.standard_normal((nb, T, shape.hidden)) * 1e-3).astype(np.float32)
    cos, sin = D.rope_cos_sin(T, shape.head_dim, shape.rope_theta, np.float32)
    K, L = shape.ckpt_interval, shape.n_layers
    t0 = time.perf_counter()
    y, _ = D.layer_forward(w, x, s1, cos, sin)          # forward
    t_fwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    _, saved = D.layer_forward(w, x, s1, cos, sin)      # recompute
    D.layer_backward(w, saved, dy, s1, cos, sin)        # backward
    t_rb = time.perf_counter() - t0
    per_layer = t_fwd * (1 + (K - 1) / K) + t_rb
    # head on the same sequence: final norm, logits, CE fwd/bwd
    Vh = shape.vocab
    wout = (rng.standard_normal((Vh, shape.hidden)) * 0.02).astype(np.float32)
    ids = rng.integers(0, Vh, (nb, T)).astype(np.int32)
    t0 = time.perf_counter()
    D.head_forward_backward(y, np.ones(shape.hidden, np.float32), wout, ids, shape.rms_eps)
    t_head = time.perf_counter() - t0
    # Adam over one layer's parameters
    n = sum(v.size for v in w.values())
    p = np.concatenate([v.reshape(-1) for v in w.values()])
    z = np.zeros_like(p)
    t0 = time.perf_counter()
    D.adam_update(p, z, z.copy(), p * 1e-3, 1, shape.lr, shape.beta1, shape.beta2, shape.adam_eps)
    t_adam_layer = time.perf_counter() - t0
    n_total = sum(int(np.prod(v)) for v in synth.param_shapes(shape).values())
    reps = shape.batch * (shape.seq // T) / nb  # samples of nb sequences per step
    step_s = reps * (L * per_layer + t_head) + t_adam_layer * n_total / n
    sample_s = t_fwd + t_rb + t_head + t_adam_layer
    return step_s, cores, sample_s, T, nb


def step_log(tag, loss, ms, st):
    log(f"{tag}: loss {loss:.4f} {ms:.0f} ms "
        f"fwd {st['fwd_ms']:.0f} head {st['head_ms']:.0f} bwd {st['bwd_ms']:.0f} "
        f"tail {st['tail_ms']:.0f} adam {st['adam_ms']:.0f} exposed "
        f"{st['exposed_wait_fwd_ms']:.0f}/{st['exposed_wait_bwd_ms']:.0f} ms; host waits "
        f"ring {st['host_ring_wait_ms']:.0f} slab {st['host_slab_wait_ms']:.0f} "
        f"op {st['host_op_wait_ms']:.0f} adam-idle {st['host_adam_idle_ms']:.0f} ms; "
        f"at {st['host_start_ms']:.0f} start, {st['gpu_done_ms']:.0f} gpu done, "
        f"{st['grads_landed_ms']:.0f} grads landed, {st['updates_done_ms']:.0f} updates done")


def gemm_layout(name):
    """NT / NN / TN from a GEMM kernel name (the layout template argument:
    first of gemm_dl_kernel, fifth of gemm_kernel)."""
    import re
    m = re.match(r"(gemm_dl_kernel|gemm_kernel)<([^>]*)>", name)
    if not m:
        return None
    args = [a.strip() for a in m.group(2).split(",")]
    lay = int(args[0] if m.group(1) == "gemm_dl_kernel" else args[4])
    return ("NT", "NN", "TN")[lay]


def kernel_table(per_step):
    """Sum each kernel's launches, time and FLOPs over the timed steps."""
    agg = {}
    for kts in per_step:
        for k in kts:
            a = agg.setdefault(k["name"], {"launches": 0, "ms": 0.0, "flops": 0.0})
            a["launches"] += k["launches"]
            a["ms"] += k["ms"]
            a["flops"] += k["flops"]
    return agg


def rate(a):
    """Achieved TFLOP/s of an aggregate: FLOPs per launch / mean launch time."""
    return a["flops"] / (a["ms"] / 1e3) / 1e12 if a["ms"] > 0 else 0.0


def run_schedule(model, shape, batches, warmup, tag, **knobs):
    """Switch the model to another schedule, then time len(batches) - warmup
    steps on a fresh arena; returns a small record."""
    import numpy as np
    import torch
    model.set_schedule(**knobs)
    torch.cuda.synchronize()
    arena = torch.empty(model.arena_bytes(shape.batch, shape.seq), dtype=torch.uint8,
                        device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    walls, stats = [], []
    for i, ids in enumerate(batches):
        ts = time.perf_counter()
        loss, st = model.step(ids, arena, streams)
        ms = 1e3 * (time.perf_counter() - ts)
        step_log(f"{tag} {'warmup' if i < warmup else 'step'} {i}", loss, ms, st)
        if i >= warmup:
            walls.append(ms)
            stats.append(st)
    torch.cuda.synchronize()
    rec = {"knobs": knobs, "steps": len(walls),
           "ms_per_step": round(float(np.mean(walls)), 2),
           "arena_bytes": int(arena.numel()),
           "exposed_wait_fwd_ms": round(float(np.mean([s["exposed_wait_fwd_ms"] for s in stats])), 2),
           "exposed_wait_bwd_ms": round(float(np.mean([s["exposed_wait_bwd_ms"] for s in stats])), 2),
           "fwd_ms": round(float(np.mean([s["fwd_ms"] for s in stats])), 2),
           "bwd_ms": round(float(np.mean([s["bwd_ms"] for s in stats])), 2),
           "h2d_bytes": float(np.mean([s["h2d_bytes"] for s in stats]))}
    del arena
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="qwen2.5-7b-b16-t1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    # weight loads in flight ahead of compute: 3 measured 1.6% faster per 7B
    # step than double buffering (1006-1009 vs 1023-1027 ms on one box)
    ap.add_argument("--prefetch-depth", type=int, default=3)
    ap.add_argument("--no-slab-pool", action="store_true")
    ap.add_argument("--ckpt-interval", type=int, default=0)
    # depth study (listing page, Table 5): the workload's width at another
    # number of layers
    ap.add_argument("--layers", type=int, default=0)
    # layers whose weights stay on the device between steps (refilled after
    # each update, during the backward): the forward streams that many fewer.
    # Default (-1): 8, at most a third of the layers.  At the 7B workload 20
    # streamed layers (8.7 ms each on the host link) plus the LM head then
    # fit within the forward's compute (about 7 ms per layer); measured
    # 0 / 8 / 12 / 16: 1060 / 1030 / 1034 / 1029 ms per step
    ap.add_argument("--resident-layers", type=int, default=-1)
    ap.add_argument("--keep-internals", type=int, default=1)
    # the hybrid 8-bit optimizer states and global-norm clipping (clipping
    # holds every gradient until the norm is known: a pool of L + 1 slabs)
    ap.add_argument("--opt-8bit", action="store_true")
    ap.add_argument("--clip-norm", type=float, default=0.0)
    # CPU threads for Adam and the embedding scatter (memory-bandwidth bound)
    ap.add_argument("--host-threads", type=int, default=16)
    # the same model under the pages' schedule after the timed steps (0: skip;
    # the default, -1, runs 3 such steps up to 64K context and none beyond,
    # where each step takes half a minute to several minutes)
    ap.add_argument("--pages-steps", type=int, default=-1)
    # the listing page's Table 4 ablation on the same model
    ap.add_argument("--ablation", action="store_true")
    # after the timed steps, three plain 1 GiB device copies: the known-size
    # kernel that hardware byte counters (rocprofv3 --pmc) are calibrated by
    ap.add_argument("--pmc-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the "
              "layer-streamed step is a single-GPU method; multi-GPU sharding is not built.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from layer_streamed_amd import metrics, mt

    shape = synth.CONFIGS[args.config]
    if args.pages_steps < 0:
        args.pages_steps = 3 if shape.seq <= 65536 else 0
    if args.ckpt_interval:
        shape = shape.with_(ckpt_interval=args.ckpt_interval)
    if args.layers:
        shape = shape.with_(n_layers=args.layers, name=f"{shape.name}-l{args.layers}")
    resident = (min(8, shape.n_layers // 3) if args.resident_layers < 0
                else min(args.resident_layers, shape.n_layers))
    keep = args.keep_internals
    torch.cuda.set_device(0)
    dev_free0, dev_total = torch.cuda.mem_get_info()
    t0 = time.perf_counter()
    model = mt.Model(shape, prefetch_depth=args.prefetch_depth,
                     use_slab_pool=0 if args.no_slab_pool else 1, check_finite=1,
                     time_kernels=1, host_threads=args.host_threads,
                     resident_layers=resident, keep_internals=keep,
                     opt_8bit=1 if args.opt_8bit else 0, clip_norm=args.clip_norm,
                     n_slabs=max(8, shape.n_layers + 1) if args.clip_norm > 0 else 8)
    log(f"model created in {time.perf_counter() - t0:.1f}s")
    t0 = time.perf_counter()
    init_weights(model, shape, seed=0)
    log(f"weights initialised in {time.perf_counter() - t0:.1f}s")
    # a fresh seeded batch for every step, drawn before any step runs
    n_batches = args.warmup + args.steps
    batches = [synth.make_tokens(shape, seed=1000 + i) for i in range(n_batches)]
    arena_bytes = model.arena_bytes(shape.batch, shape.seq)
    arena = torch.empty(arena_bytes, dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    for i in range(args.warmup):
        t0 = time.perf_counter()
        loss, st = model.step(batches[i], arena, streams)
        step_log(f"warmup {i}", loss, 1e3 * (time.perf_counter() - t0), st)
    torch.cuda.synchronize()
    stats, losses, step_wall, ktimes = [], [], [], []
    t_start = time.perf_counter()
    for i in range(args.steps):
        ts = time.perf_counter()
        loss, st = model.step(batches[args.warmup + i], arena, streams)
        step_wall.append(1e3 * (time.perf_counter() - ts))
        stats.append(st)
        losses.append(loss)
        ktimes.append(model.kernel_times())
        step_log(f"step {i}", loss, step_wall[-1], st)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = 1e3 * elapsed / args.steps
    # device memory the process holds beyond what it held before the model
    # existed: the arena plus the library's own (events, static scratch)
    dev_used = dev_free0 - torch.cuda.mem_get_info()[0]
    log(f"dominant kernel per step: {[s['probe_kernel'] for s in stats]}")
    del arena
    torch.cuda.empty_cache()

    n_params = metrics.shape_param_count(shape)
    D = shape.tokens
    f_formula = metrics.formula_flops(n_params, shape.n_layers, shape.hidden, shape.batch, shape.seq)
    f_xb = metrics.formula_flops_xbatch(n_params, shape.n_layers, shape.hidden, shape.batch, shape.seq)
    _, plan_ops, _, _ = mt.debug_plan(shape.n_layers, shape.ckpt_interval, args.prefetch_depth,
                                      keep, resident)
    f_exec = metrics.executed_flops(shape, plan_ops, keep)
    f_timed = float(np.mean([s["probe_all_flops"] for s in stats]))
    step_s = ms_per_step / 1e3
    tflops = f_formula / step_s / 1e12
    tok_s = D / step_s

    # per-kernel aggregates over the timed steps; the dominant kernel is the
    # one with the largest total time
    agg = kernel_table(ktimes)
    kernel = max(agg, key=lambda k: agg[k]["ms"]) if agg else ""
    top = agg.get(kernel, {"launches": 0, "ms": 0.0, "flops": 0.0})
    probe_n = top["launches"]
    avg_launch_ms = top["ms"] / max(probe_n, 1)
    flops_per_launch = top["flops"] / max(probe_n, 1)
    achieved = rate(top)
    gemm_ms = float(np.mean([s["probe_all_gemm_ms"] for s in stats]))
    attn_ms = float(np.mean([s["probe_all_attn_ms"] for s in stats]))
    families = {}
    for name, a in agg.items():
        lay = gemm_layout(name)
        if lay:
            f = families.setdefault(lay, {"launches": 0, "ms": 0.0, "flops": 0.0})
            for k in f:
                f[k] += a[k]
    gemm_families = {lay: {"ms_per_step": round(f["ms"] / args.steps, 2),
                           "tflops": round(rate(f), 1),
                           "frac": round(rate(f) / PEAK_BF16_TFLOPS, 4)}
                     for lay, f in sorted(families.items())}
    attn = {}
    for name, a in agg.items():
        if name.startswith("attn"):
            attn[name] = {"ms_per_step": round(a["ms"] / args.steps, 3),
                          "avg_launch_ms": round(a["ms"] / max(a["launches"], 1), 4),
                          "tflops": round(rate(a), 1),
                          "frac": round(rate(a) / PEAK_BF16_TFLOPS, 4)}
    # the backward as a whole against its 5 algorithmic products (the two
    # kernels together execute 7: S and dP are formed in both)
    bwd = [a for n, a in agg.items() if n.startswith(("attn_delta", "attn_dkdv", "attn_dq"))]
    if bwd:
        b_ms = sum(a["ms"] for a in bwd)
        b_alg = sum(a["flops"] for a in bwd) * 5 / 7
        attn["backward_algorithmic"] = {
            "ms_per_step": round(b_ms / args.steps, 3),
            "tflops": round(b_alg / (b_ms / 1e3) / 1e12, 1),
            "frac": round(b_alg / (b_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    h2d = np.mean([s["h2d_bytes"] for s in stats])
    d2h = np.mean([s["d2h_bytes"] for s in stats])
    h2d_ms = np.mean([s["h2d_ms"] for s in stats])
    d2h_ms = np.mean([s["d2h_ms"] for s in stats])

    # the pages' schedule on the same model: every layer streamed every
    # step (no resident layers), double buffering, and the per-layer
    # recompute inside the backward instead of kept internals
    pages = None
    base_knobs = dict(prefetch_depth=args.prefetch_depth, resident_layers=resident,
                      keep_internals=keep, use_slab_pool=0 if args.no_slab_pool else 1,
                      ckpt_interval=shape.ckpt_interval)
    if args.pages_steps > 0:
        pb = [synth.make_tokens(shape, seed=2000 + i) for i in range(1 + args.pages_steps)]
        pages = run_schedule(model, shape, pb, 1, "pages",
                             prefetch_depth=2, resident_layers=0, keep_internals=0)
        pages["tflops"] = round(f_formula / (pages["ms_per_step"] / 1e3) / 1e12, 3)
        pages["tokens_per_s"] = round(D / (pages["ms_per_step"] / 1e3), 1)
    ablation = None
    if args.ablation:
        # listing page, Table 4: double buffering off (depth 1), slab pool
        # off, checkpoint interval 1; each against the pages' schedule and
        # the tuned one
        pages_k = dict(prefetch_depth=2, resident_layers=0, keep_internals=0, use_slab_pool=1,
                       ckpt_interval=shape.ckpt_interval)
        variants = [
            ("pages", pages_k),
            ("pages, no double buffering", dict(pages_k, prefetch_depth=1)),
            ("pages, no slab pool", dict(pages_k, use_slab_pool=0)),
            ("pages, K=1", dict(pages_k, ckpt_interval=1)),
            ("tuned", dict(base_knobs, use_slab_pool=1)),
            ("tuned, recompute (keep_internals=0)", dict(base_knobs, use_slab_pool=1,
                                                          keep_internals=0)),
            ("tuned, no resident layers", dict(base_knobs, use_slab_pool=1, resident_layers=0)),
            ("tuned, depth 2", dict(base_knobs, use_slab_pool=1, prefetch_depth=2)),
            ("tuned, no slab pool", dict(base_knobs, use_slab_pool=0)),
            ("tuned, K=1", dict(base_knobs, use_slab_pool=1, ckpt_interval=1)),
        ]
        ablation = []
        for j, (label, kn) in enumerate(variants):
            if args.no_slab_pool and kn.get("use_slab_pool"):
                continue
            ab = [synth.make_tokens(shape, seed=3000 + 10 * j + i) for i in range(3)]
            r = run_schedule(model, shape, ab, 1, label, **kn)
            r["label"] = label
            r["tflops"] = round(f_formula / (r["ms_per_step"] / 1e3) / 1e12, 3)
            ablation.append(r)
            log(f"ablation {label}: {r['ms_per_step']:.0f} ms/step, {r['tflops']:.1f} TFLOPS, "
                f"arena {r['arena_bytes'] / 2**30:.2f} GiB")

    if args.pmc_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # the host link's copy rate in this run, after the timed steps: three
    # 1 GiB pinned <-> device copies each way (not under --pmc-copy, whose
    # counter passes calibrate on the device copy alone)
    link_peak = {}
    hbuf = None
    if not args.pmc_copy:
        try:
            hbuf = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
        except RuntimeError as e:  # the wide models pin most of what the host allows
            log(f"link copy rate not measured: pinning 1 GiB failed ({e})")
    if hbuf is not None:
        dbuf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        for name, dst, src in (("h2d", dbuf, hbuf), ("d2h", hbuf, dbuf)):
            dst.copy_(src, non_blocking=True)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                dst.copy_(src, non_blocking=True)
            e1.record()
            torch.cuda.synchronize()
            link_peak[name] = 3 * (1 << 30) / (e0.elapsed_time(e1) / 1e3) / 1e9
        del hbuf, dbuf

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        cpu_step_s, cores, sample_s, T_s, nb_s = cpu_baseline(shape)
        log(f"cpu baseline: {cpu_step_s:.0f} s/step extrapolated from a {sample_s:.1f} s sample "
            f"({time.perf_counter() - t0:.1f} s with weight draws)")
        cpu = {
            "value": round(f_formula / cpu_step_s / 1e12, 4),
            "unit": "TFLOPS (6ND+12LHT^2)",
            "tokens_per_s": round(D / cpu_step_s, 3),
            "cores": int(cores),
            "kind": "oracle",
            "sample": (f"one decoder layer at the full width on {nb_s} x {T_s} tokens "
                       f"(forward, re-forward share, recompute, backward) + head on the same "
                       f"tokens + Adam over one layer ({sample_s:.1f} s of CPU work); "
                       f"extrapolated x{shape.n_layers} layers x "
                       f"{shape.batch * (shape.seq // T_s) / nb_s:g} samples"),
        }

    line = {
        "metric": "sustained TFLOPS (6ND+12LHT^2) + tokens/s, Qwen2.5-7B-shaped streamed step",
        "value": round(tflops, 3),
        "unit": "TFLOPS",
        "tokens_per_s": round(tok_s, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded uniform token ids, a fresh batch each step; random init)",
        "config": {
            "workload": shape.name,
            "layers": shape.n_layers, "hidden": shape.hidden, "heads": shape.n_heads,
            "kv_heads": shape.n_kv_heads, "ffn": shape.ffn, "vocab": shape.vocab,
            "global_batch": shape.batch, "seq_len": shape.seq,
            "ckpt_interval": shape.ckpt_interval, "prefetch_depth": args.prefetch_depth,
            "slab_pool": not args.no_slab_pool,
            "resident_layers": resident,
            "keep_internals": keep,
            "opt_8bit": bool(args.opt_8bit),
            "clip_norm": args.clip_norm,
            "parallelism": "single-gpu layer streaming",
            "params": n_params,
        },
        "step_ms": {"median": round(float(np.median(step_wall)), 2),
                    "min": round(float(np.min(step_wall)), 2),
                    "max": round(float(np.max(step_wall)), 2)},
        "tflops_xbatch_formula": round(f_xb / step_s / 1e12, 3),
        # FLOPs the step's plan executes (forward, re-forward, recompute if
        # any, backward, head; attention by causal pairs), and the same
        # summed over the timed launches themselves
        "executed_tflop_per_step": round(f_exec / 1e12, 2),
        "timed_launch_tflop_per_step": round(f_timed / 1e12, 2),
        "tflops_executed": round(f_exec / step_s / 1e12, 3),
        "mfma_frac_executed": round(f_exec / step_s / 1e12 / PEAK_BF16_TFLOPS, 4),
        "phases_ms": {k: round(float(np.mean([s[k] for s in stats])), 2) for k in
                      ("fwd_ms", "head_ms", "bwd_ms", "tail_ms", "adam_ms",
                       "exposed_wait_fwd_ms", "exposed_wait_bwd_ms", "host_ring_wait_ms",
                       "host_slab_wait_ms", "host_op_wait_ms", "host_adam_idle_ms",
                       "host_start_ms", "gpu_done_ms", "grads_landed_ms", "updates_done_ms")},
        "link": {"h2d_bytes": h2d, "d2h_bytes": d2h,
                 "h2d_GBps_while_copying": round(h2d / max(h2d_ms, 1e-9) / 1e6, 2),
                 "d2h_GBps_while_copying": round(d2h / max(d2h_ms, 1e-9) / 1e6, 2),
                 "h2d_GBps_per_step": round(h2d / step_s / 1e9, 2),
                 "d2h_GBps_per_step": round(d2h / step_s / 1e9, 2),
                 # the same run's 1 GiB pinned copies, and PCIe Gen5 x16 per
                 # direction (32 GT/s x 16 lanes x 128/130 / 8)
                 "h2d_peak_GBps": round(link_peak["h2d"], 2) if link_peak else None,
                 "d2h_peak_GBps": round(link_peak["d2h"], 2) if link_peak else None,
                 "h2d_busy_frac_of_peak": (round(h2d / step_s / 1e9 / link_peak["h2d"], 3)
                                           if link_peak else None),
                 "d2h_busy_frac_of_peak": (round(d2h / step_s / 1e9 / link_peak["d2h"], 3)
                                           if link_peak else None),
                 "nominal_GBps": 63.0},
        "host_bytes": {"pinned": stats[-1]["pinned_host_bytes"],
                       "pageable": stats[-1]["pageable_host_bytes"]},
        "device_arena_bytes": stats[-1]["device_arena_bytes"],
        "device_used_bytes": int(dev_used),
        "loss": losses[-1],
        "grad_norm": stats[-1]["grad_norm"],
        "clip_factor": stats[-1]["clip_factor"],
        "gemm_ms_per_step": round(gemm_ms, 2),
        "attn_ms_per_step": round(attn_ms, 2),
        "gemm_families": gemm_families,
        "attention": attn,
        "roofline": {
            "kernel": kernel,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": (measured_traffic(kernel)
                        if shape.name == "qwen2.5-7b-b16-t1024" else None),
            "avg_launch_ms": round(avg_launch_ms, 4),
            "flops_per_launch": flops_per_launch,
            "launches": probe_n,
        },
        "pages_schedule": pages,
        "cpu_baseline": cpu,
    }
    if ablation is not None:
        line["ablation"] = ablation
    model.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
