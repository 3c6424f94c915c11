"""Benchmark of the layer-streamed training step on one MI355X.

Workload (default): Qwen2.5-7B-shaped decoder, random N(0, 0.02^2) init,
batch 16 x seq 1024 uniform random token ids, checkpoint interval 4; bf16
weights stream from pinned host memory, fp32 master + Adam states on the
host, CPU Adam, weight loads up to 3 layers ahead of compute.  Layers 1-8
(at most a third of the layers) stay on the device between steps: each
one's updated copy streams in during the backward right after its host
update (--resident-layers).  A step is one full mt_stream_step (forward,
head, segment re-forward, recompute + backward, gradient offload, CPU Adam
of every unit).

Prints one JSON line: sustained TFLOPS by the 6ND + 12LHT^2 formula
(MegaTrain listing page, Table 7 caption; T^2 term not scaled by the batch)
plus tokens/s, the roofline of the dominant kernel (the GEMM kernel
instantiation with the largest total time in the step, every launch timed
with HIP events on the compute stream inside the timed steps), and the CPU
oracle timed on a bounded sample.
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
    # layers whose weights stay on the device between steps (refilled after
    # each update, during the backward): the forward streams that many fewer.
    # Default (-1): 8, at most a third of the layers.  At the 7B workload 20
    # streamed layers (8.7 ms each on the host link) plus the LM head then
    # fit within the forward's compute (about 7 ms per layer); measured
    # 0 / 8 / 12 / 16: 1060 / 1030 / 1034 / 1029 ms per step
    ap.add_argument("--resident-layers", type=int, default=-1)
    # CPU threads for Adam and the embedding scatter (memory-bandwidth bound)
    ap.add_argument("--host-threads", type=int, default=16)
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
    if args.ckpt_interval:
        shape = shape.with_(ckpt_interval=args.ckpt_interval)
    resident = (min(8, shape.n_layers // 3) if args.resident_layers < 0
                else min(args.resident_layers, shape.n_layers))
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    model = mt.Model(shape, prefetch_depth=args.prefetch_depth,
                     use_slab_pool=0 if args.no_slab_pool else 1, check_finite=1,
                     time_kernels=1, host_threads=args.host_threads,
                     resident_layers=resident)
    log(f"model created in {time.perf_counter() - t0:.1f}s")
    t0 = time.perf_counter()
    init_weights(model, shape, seed=0)
    log(f"weights initialised in {time.perf_counter() - t0:.1f}s")
    ids = synth.make_tokens(shape)
    arena_bytes = model.arena_bytes(shape.batch, shape.seq)
    arena = torch.empty(arena_bytes, dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    for i in range(args.warmup):
        t0 = time.perf_counter()
        loss, st = model.step(ids, arena, streams)
        log(f"warmup {i}: loss {loss:.4f} {1e3 * (time.perf_counter() - t0):.0f} ms")
    torch.cuda.synchronize()
    stats = []
    losses = []
    step_wall = []
    t_start = time.perf_counter()
    for i in range(args.steps):
        ts = time.perf_counter()
        loss, st = model.step(ids, arena, streams)
        step_wall.append(1e3 * (time.perf_counter() - ts))
        stats.append(st)
        losses.append(loss)
        log(f"step {i}: loss {loss:.4f} {1e3 * (time.perf_counter() - ts):.0f} ms "
            f"fwd {st['fwd_ms']:.0f} head {st['head_ms']:.0f} bwd {st['bwd_ms']:.0f} "
            f"tail {st['tail_ms']:.0f} adam {st['adam_ms']:.0f} exposed "
            f"{st['exposed_wait_fwd_ms']:.0f}/{st['exposed_wait_bwd_ms']:.0f} ms; host waits "
            f"ring {st['host_ring_wait_ms']:.0f} slab {st['host_slab_wait_ms']:.0f} "
            f"op {st['host_op_wait_ms']:.0f} adam-idle {st['host_adam_idle_ms']:.0f} ms; "
            f"at {st['host_start_ms']:.0f} start, {st['gpu_done_ms']:.0f} gpu done, "
            f"{st['grads_landed_ms']:.0f} grads landed, {st['updates_done_ms']:.0f} updates done")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = 1e3 * elapsed / args.steps
    log(f"dominant GEMM kernel per step: {[s['probe_kernel'] for s in stats]}")
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
    if not args.pmc_copy:
        hbuf = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
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

    n_params = metrics.shape_param_count(shape)
    D = shape.tokens
    f_formula = metrics.formula_flops(n_params, shape.n_layers, shape.hidden, shape.batch, shape.seq)
    f_xb = metrics.formula_flops_xbatch(n_params, shape.n_layers, shape.hidden, shape.batch, shape.seq)
    f_exec = metrics.executed_flops(shape)
    step_s = ms_per_step / 1e3
    tflops = f_formula / step_s / 1e12
    tok_s = D / step_s

    # the GEMM kernel instantiation with the largest total time (per step,
    # from HIP events on the compute stream); the one most steps name
    names = [s["probe_kernel"] for s in stats]
    kernel = max(set(names), key=names.count) if names else ""
    kstats = [s for s in stats if s["probe_kernel"] == kernel]
    probe_ms = sum(s["probe_kernel_ms"] for s in kstats)
    probe_n = sum(s["probe_kernel_launches"] for s in kstats)
    probe_flops = sum(s["probe_kernel_flops"] for s in kstats)
    gemm_ms = float(np.mean([s["probe_all_gemm_ms"] for s in stats]))
    avg_launch_ms = probe_ms / max(probe_n, 1)
    flops_per_launch = probe_flops / max(probe_n, 1)
    achieved = flops_per_launch / (avg_launch_ms / 1e3) / 1e12 if probe_n else 0.0
    h2d = np.mean([s["h2d_bytes"] for s in stats])
    d2h = np.mean([s["d2h_bytes"] for s in stats])
    h2d_ms = np.mean([s["h2d_ms"] for s in stats])
    d2h_ms = np.mean([s["d2h_ms"] for s in stats])

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
        "data": "synthetic",
        "config": {
            "workload": shape.name,
            "layers": shape.n_layers, "hidden": shape.hidden, "heads": shape.n_heads,
            "kv_heads": shape.n_kv_heads, "ffn": shape.ffn, "vocab": shape.vocab,
            "global_batch": shape.batch, "seq_len": shape.seq,
            "ckpt_interval": shape.ckpt_interval, "prefetch_depth": args.prefetch_depth,
            "slab_pool": not args.no_slab_pool,
            "resident_layers": resident,
            "parallelism": "single-gpu layer streaming",
            "params": n_params,
        },
        "step_ms": {"median": round(float(np.median(step_wall)), 2),
                    "min": round(float(np.min(step_wall)), 2),
                    "max": round(float(np.max(step_wall)), 2)},
        "tflops_xbatch_formula": round(f_xb / step_s / 1e12, 3),
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
        "loss": losses[-1],
        "gemm_ms_per_step": round(gemm_ms, 2),
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
        "cpu_baseline": cpu,
    }
    model.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
