"""Benchmark: one MoE expert-layer forward per step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral]

A step is the whole hot path on one batch of synthetic tokens that is
already resident in HBM: route -> permute -> (shared experts) -> grouped
GEMM0 + SwiGLU (token rows gathered on load) -> grouped GEMM1 -> weighted
combine.  The default
workload is the Mixtral-8x7B-shape layer (T=4096, d=4096, f=14336, E=8,
top-2, bf16).  Prints one JSON line with the layer's throughput in TFLOP/s
(algorithmic flops, no padding), tokens/s, the per-stage times from HIP
events recorded on the launch stream, the roofline of the dominant kernel
(the layer-0 grouped GEMM) and the fp64 CPU oracle timed on a bounded token
sample of the same layer on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE layer fwd TFLOP/s (% bf16 MFMA peak) + tokens/s, 1×MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--path", default="fast", choices=["fast", "fast32", "atomic", "reference"],
                    help="fast: gather fused into layer 0, separate deterministic combine over "
                         "compact rows (fp16 + a power-of-two factor per 32 columns); "
                         "fast32: the same over fp32 rows; "
                         "atomic: combine fused into layer 1 with atomic adds; "
                         "reference: permuted copy of x and separate combine")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--protocol-steps", type=int, default=20,
                    help="steps of the cache-flushed per-step timing (median, p10, p90)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured peaks (MFMA-only loop, 1 GiB device copy)")
    ap.add_argument("--cpu-target-s", type=float, default=10.0,
                    help="approximate seconds of oracle work for the CPU baseline sample")
    ap.add_argument("--sweep", choices=["tokens", "skew"], default=None,
                    help="instead of one workload, time the Mixtral-shape layer over the "
                         "token-count sweep (T = 128 .. 32768) or the router-bias-strength "
                         "sweep (0 .. 2x the skewed workload's bias); one JSON line per point")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step instead: the forward that keeps h = x W_gate and "
                         "u = x W_up, then the backward of a seeded upstream gradient; one JSON "
                         "line with the backward's rate and per-stage times")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the layer, run a plain device copy of BYTES bytes three "
                         "times (the reference reading for HBM byte counters)")
    return ap.parse_args()


def copy_calibration(nbytes):
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 3}), flush=True)


def stage_bytes(cfg, compact=False):
    """Algorithmic HBM bytes of the memory-bound stages of the fused path:
    route = x once, W_r once, the top-k indices and weights out; permute =
    the indices and weights in, perm_token, inv and perm_w out (the gather
    is fused into layer 0); combine = the k expert rows of every token in
    (fp32, or compact: fp16 plus one fp32 factor per 32 columns), y out, the
    indices and weights in, plus the shared-expert output in the same form
    (and its gate logit) when the layer has shared experts."""
    s = 2 if cfg.dtype == "bf16" else 4
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    R = T * k
    row = d * 2 + d // 32 * 4 if compact else d * 4  # one expert row as the combine reads it
    comb = R * row + T * d * 4 + T * k * 8
    if cfg.n_shared:
        comb += T * row + (T * 4 if cfg.shared_gated else 0)
    return {
        "route": T * d * s + d * E * s + T * k * 8,
        "permute": R * 4 + R * 4 + 3 * R * 4,
        "combine": comb,
    }


def pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v), q))


def protocol_times(m, steps, flush_bytes):
    """Per-step HIP-event times of `steps` layer steps, each preceded by a
    write of `flush_bytes` bytes (outside the events) that evicts the 256 MB
    last-level cache, so no stage finds its inputs cached from the previous
    step.  Returns {stage: [ms per step]} and the whole steps' ms."""
    import torch
    stream = torch.cuda.current_stream()
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda:0")
    stages = m.STAGES
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(steps)]
    for s in range(steps):
        flush.fill_(s & 0xFF)
        ev[s][0].record(stream)
        pos = [1]

        def mark(_name, s=s, pos=pos):
            ev[s][pos[0]].record(stream)
            pos[0] += 1

        m.forward(marks=mark)
    torch.cuda.synchronize()
    per = {name: [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]
           for i, name in enumerate(stages)}
    step = [ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)]
    del flush
    return per, step


def flushed_read_ms(nbytes, reps=5, flush_bytes=1 << 30):
    """Median HIP-event time of a pure streaming read (moe_probe_read) of
    `nbytes` bytes, each rep after a write of `flush_bytes` bytes that evicts
    the last-level cache (outside the events)."""
    import torch
    from mixture_experts_layer_top_amd import _lib
    nbytes = (nbytes + 15) // 16 * 16
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda:0")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _lib.moe_probe_read(src, nbytes, sink)  # warm-up
    times = []
    for r in range(reps):
        flush.fill_(r & 0xFF)
        a.record()
        _lib.moe_probe_read(src, nbytes, sink)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del src, flush
    return sorted(times)[reps // 2]


def measured_peaks(copy_bytes=1 << 30, probe_iters=2500, probe_launches=20):
    """Peaks measured on this machine: the bf16 MFMA rate and shader clock of an
    all-compute-unit MFMA-only loop (two 4-wave blocks per compute unit), with
    operands that change from one MFMA to the next (random bf16 values, as in
    a GEMM) and with fixed operands, each timed over `probe_launches` launches
    after as many warm-up launches (the clock settles over tens of
    milliseconds of load); and a device copy of `copy_bytes` bytes (read +
    write bytes / time)."""
    import torch
    from mixture_experts_layer_top_amd import _lib
    dev = torch.device("cuda:0")
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * n_cu
    ticks = torch.zeros(3 * blocks, dtype=torch.int64, device=dev)
    g = torch.Generator(device=dev).manual_seed(0)
    ops = torch.randn(blocks * 16 * 256 * 8, generator=g, device=dev).to(torch.bfloat16)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def mfma_rate(operands):
        for _ in range(probe_launches):  # warm-up
            _lib.moe_probe_mfma(blocks, probe_iters, operands, ticks)
        a.record()
        for _ in range(probe_launches):
            _lib.moe_probe_mfma(blocks, probe_iters, operands, ticks)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        flops = probe_launches * blocks * 4 * probe_iters * 32 * 16384
        t = ticks.view(blocks, 3).cpu().double()  # the last launch
        sclk = float((t[:, 0] / (t[:, 1] / 100e6)).median()) / 1e9
        return flops / (ms * 1e-3) / 1e12, sclk, ms

    rnd_tf, rnd_clk, rnd_ms = mfma_rate(ops)
    fix_tf, fix_clk, _ = mfma_rate(None)
    del ops
    src = torch.empty(copy_bytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del src, dst
    cms = sorted(times)[len(times) // 2]
    return {
        "mfma_bf16_TFLOPs": round(rnd_tf, 1),
        "sclk_GHz_under_mfma_load": round(rnd_clk, 3),
        "mfma_bf16_TFLOPs_fixed_operands": round(fix_tf, 1),
        "sclk_GHz_fixed_operands": round(fix_clk, 3),
        "mfma_probe": f"{probe_launches} launches of {blocks} blocks x 4 waves x {probe_iters} x 32 "
                      f"MFMA 16x16x32 bf16 after {probe_launches} warm-up launches, random bf16 "
                      f"operands changing every MFMA ({rnd_ms:.1f} ms); the same with fixed "
                      "operands",
        "hbm_copy_GBs": round(2 * copy_bytes / (cms * 1e-3) / 1e9, 1),
        "copy": f"device copy of {copy_bytes >> 20} MiB, median of 5",
        "hbm_read_GBs": round(copy_bytes / (flushed_read_ms(copy_bytes) * 1e-3) / 1e9, 1),
        "read": f"streaming read (moe_probe_read) of {copy_bytes >> 20} MiB after a 1 GiB "
                "flush, median of 5",
    }


def gemm_kernel_name(cfg, up):
    """The grouped-GEMM kernel the library launches for this layer: for bf16
    the ping-pong kernel (main pass) when K is a multiple of its 64-deep
    stages and the A operand is below 4 GiB, in the instantiation that may
    hold wide items (an expert's last rows over two N panels) when K >= 2048,
    else the general kernel; for fp32 the plain FMA kernels."""
    if cfg.dtype != "bf16":
        return "up_f32_kernel" if up else "down_f32_kernel"
    K = cfg.d if up else cfg.f
    a_bytes = cfg.T * cfg.k * K * 2
    u = "true" if up else "false"
    if K % 64 == 0 and a_bytes < (1 << 32):
        wide = "true" if K >= 2048 else "false"
        return f"grouped_gemm_bf16_pp_kernel<{u}, 64, false, {wide}>"
    return f"grouped_gemm_bf16_kernel<{u}, 2, 4, 256>"


def measured_traffic(cfg):
    """HBM bytes per launch of the layer-0 GEMM from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None when gemm.hip has changed since the
    counters were taken (or they were taken on another workload)."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(HERE, "profiles", "gemm_up_traffic.json")))
        src = open(os.path.join(HERE, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest()[:16] != rec["source_sha256_16"]:
        return None
    if not rec["workload"].startswith(cfg.name + " "):
        return None
    if rec["kernel"] != gemm_kernel_name(cfg, up=True):
        return None
    return rec["traffic_bytes"]


def route_alone(m, reps=20, flush_bytes=1 << 30):
    """The router call on its own: `reps` calls back to back (one event pair
    around them), and `reps` single calls each after a 1 GiB write that
    evicts the last-level cache (median of the per-call event times)."""
    import torch
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m.route()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        m.route()
    b.record(stream)
    torch.cuda.synchronize()
    b2b = a.elapsed_time(b) / reps
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda:0")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i in range(reps):
        flush.fill_(i & 0xFF)
        ev[i][0].record(stream)
        m.route()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    del flush
    return b2b, pct([x.elapsed_time(y) for x, y in ev], 50)


def cpu_routing(cfg, layer, target_s=3.0):
    """The oracle's routing and dispatch alone (logits, top-k, weights,
    counts, offsets, stable permutation) on all T tokens, fp64 numpy: the
    CPU counterpart of the route and permute calls.  Seconds per call
    (median of the repetitions that fit in about target_s seconds)."""
    import oracle.moe_oracle as O
    from mixture_experts_layer_top_amd.inputs import to_f64
    host = to_f64({kk: layer[kk] for kk in ("x", "W_r", "b") if layer.get(kk) is not None})
    times = []
    while sum(times) < target_s and len(times) < 20:
        t0 = time.perf_counter()
        _, idx, w = O.route(host, cfg.k, cfg.renorm)
        O.dispatch(idx, w, cfg.E)
        times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2], len(times)


def cpu_baseline(cfg, layer, target_s):
    """The fp64 oracle, as it stands, on a bounded sample of the workload's
    tokens with the full expert weights (the same tensors the GPU ran on;
    the bf16 -> fp64 conversion is excluded from the time)."""
    from threadpoolctl import threadpool_info
    import oracle.moe_oracle as O
    from mixture_experts_layer_top_amd.inputs import to_f64

    host = to_f64(layer)
    # grow the token sample 4x at a time until one forward takes >= target/4
    # (or the whole batch is reached), then repeat that sample until about
    # target_s seconds of oracle work have been timed
    n = 64
    while True:
        sub = dict(host, x=host["x"][:n])
        t0 = time.perf_counter()
        O.forward(sub, cfg.k, cfg.renorm)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or n >= cfg.T:
            break
        n = min(cfg.T, n * 4)
    reps, total = 1, dt
    while total < target_s:
        t0 = time.perf_counter()
        O.forward(sub, cfg.k, cfg.renorm)
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    sub_cfg = cfg.shrink(T=n, d=cfg.d, f=cfg.f, f_shared=cfg.f_shared)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    del host
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": sub_cfg.flops() / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {n} of {cfg.T} tokens, full expert weights, fp64 numpy; "
                  f"{reps} forward(s), {dt:.2f} s each; bf16->fp64 input conversion excluded",
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": model,
    }


def time_layer(cfg, args):
    """Draw the layer on the GPU, run the warmup steps, then time exactly
    args.steps steps (host sync on both sides; one event pair around them on
    the launch stream), then run args.steps more with HIP events between
    stages for the per-stage times.  Returns the layer, the MoeLayer, the
    wall-clock ms per step, the event ms per step and the per-stage ms."""
    import torch
    from mixture_experts_layer_top_amd.inputs import make_layer
    from mixture_experts_layer_top_amd.layer import MoeLayer

    dev = torch.device("cuda:0")
    layer = make_layer(cfg, seed=0, device=dev)
    m = MoeLayer(cfg, layer, keep_logits=False, path=args.path)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        m.forward()
    torch.cuda.synchronize()

    # the timed steps: nothing but the layer between the two syncs (one
    # event pair around all of them gives the GPU-side time per step)
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for s in range(args.steps):
        m.forward()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e_start.elapsed_time(e_end) / args.steps

    # per-stage times from as many further steps, with an event on the
    # stream after every stage (each event record costs a few microseconds
    # of GPU time, so these steps are not the timed ones)
    stages = MoeLayer.STAGES
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    for s in range(args.steps):
        ev[s][0].record(stream)
        pos = [1]

        def mark(_name, s=s, pos=pos):
            ev[s][pos[0]].record(stream)
            pos[0] += 1

        m.forward(marks=mark)
    torch.cuda.synchronize()
    stage_ms = {}
    for i, name in enumerate(stages):
        stage_ms[name] = sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
    return layer, m, wall * 1e3 / args.steps, step_ms, stage_ms


def run_sweep(args):
    """One JSON line per point of the token-count or router-bias sweep of the
    Mixtral-shape layer (the robustness axes of the COMET page, "COMET's
    Performance": input token length and imbalanced expert loads)."""
    import torch
    from mixture_experts_layer_top_amd.inputs import sweep_configs

    for cfg in sweep_configs(args.sweep):
        layer, m, ms_per_step, step_ms, stage_ms = time_layer(cfg, args)
        counts = m.counts.cpu().numpy()
        share = counts / max(1, counts.sum())
        T, d, f, k = cfg.T, cfg.d, cfg.f, cfg.k
        R = T * k
        out = {
            "metric": METRIC,
            "sweep": args.sweep,
            "workload": cfg.name,
            "T": T, "d": d, "f": f, "E": cfg.E, "k": k,
            "bias_scale": cfg.bias_scale if cfg.biased else 0.0,
            "value": round(cfg.flops() / (ms_per_step * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s",
            "ms_per_step": round(ms_per_step, 4),
            "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
            "steps": args.steps, "warmup": args.warmup,
            "expert_share_max": round(float(share.max()), 4),
            "expert_share_min": round(float(share.min()), 4),
            "stages_ms": {kk: round(v, 4) for kk, v in stage_ms.items()},
            "expert_up_TFLOPs": round(4 * R * d * f / (stage_ms["expert_up"] * 1e-3) / 1e12, 1),
            "expert_down_TFLOPs": round(2 * R * f * d / (stage_ms["expert_down"] * 1e-3) / 1e12, 1),
        }
        print(json.dumps(out), flush=True)
        del layer, m
        torch.cuda.empty_cache()


def backward_flops(cfg):
    """Algorithmic flops of the layer's backward: each GEMM's data and weight
    gradients (twice the forward's GEMM flops), the router's dW_r and dx
    (2 * 2 T d E) and the shared gate's (2 * 2 T d)."""
    T, d, f, E, k = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k
    fl = 12 * T * k * d * f + 4 * T * d * E
    fl += cfg.n_shared * 12 * T * d * cfg.f_shared
    if cfg.shared_gated:
        fl += 4 * T * d
    return fl


def run_backward(args):
    """Training step of the workload: forward (train=True) then backward, the
    backward's stages bracketed by HIP events on the launch stream."""
    import torch
    from mixture_experts_layer_top_amd.inputs import CONFIGS, make_layer
    from mixture_experts_layer_top_amd.layer import MoeLayer

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    layer = make_layer(cfg, seed=0, device=dev)
    if args.path not in ("fast", "fast32", "reference"):
        raise SystemExit(f"--backward trains a separate combine: --path {args.path} has none")
    m = MoeLayer(cfg, layer, path=args.path, train=True)
    dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator(device=dev).manual_seed(1),
                     device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        m.forward()
        m.backward(dy)
    torch.cuda.synchronize()
    bst = MoeLayer.BSTAGES
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(bst) + 2)]
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        m.forward()
        ev[s][1].record(stream)
        pos = [2]

        def mark(_name, s=s, pos=pos):
            ev[s][pos[0]].record(stream)
            pos[0] += 1

        m.backward(dy, marks=mark)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg = lambda i, j: sum(ev[s][i].elapsed_time(ev[s][j]) for s in range(args.steps)) / args.steps  # noqa: E731
    fwd_ms = avg(0, 1)
    bwd_ms = avg(1, len(bst) + 1)
    stage_ms = {name: avg(i + 1, i + 2) for i, name in enumerate(bst)}
    T, d, f, k = cfg.T, cfg.d, cfg.f, cfg.k
    R = T * k
    out = {
        "metric": "MoE layer bwd TFLOP/s + training-step tokens/s, 1xMI355X",
        "workload": cfg.name, "T": T, "d": d, "f": f, "E": cfg.E, "k": k,
        "path": args.path, "combine": m.comb,
        "value": round(backward_flops(cfg) / (bwd_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "steps": args.steps, "warmup": args.warmup,
        "train_step_ms": round(wall * 1e3 / args.steps, 4),
        "train_tokens_per_s": round(T / (wall / args.steps), 1),
        "forward_ms": round(fwd_ms, 4), "backward_ms": round(bwd_ms, 4),
        "backward_stages_ms": {kk: round(v, 4) for kk, v in stage_ms.items()},
        "stage_rates": {
            "expert_down_bwd_TFLOPs": round(4 * R * d * f / (stage_ms["expert_down_bwd"] * 1e-3) / 1e12, 1),
            "expert_up_bwd_TFLOPs": round(8 * R * d * f / (stage_ms["expert_up_bwd"] * 1e-3) / 1e12, 1),
        },
        "dtype": "bf16", "data": "synthetic",
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the expert layer is timed on one GPU's share "
              "of tokens, and no multi-GPU path exists in this build (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    from mixture_experts_layer_top_amd.inputs import CONFIGS
    from mixture_experts_layer_top_amd import _lib

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    _lib.load()
    if args.sweep:
        run_sweep(args)
        return
    if args.backward:
        run_backward(args)
        return
    cfg = CONFIGS[args.workload]
    layer, m, ms_per_step, step_ms, stage_ms = time_layer(cfg, args)

    flops = cfg.flops()
    T, d, f, k = cfg.T, cfg.d, cfg.f, cfg.k
    R = T * k
    g0_flops = 4 * R * d * f
    g1_flops = 2 * R * f * d
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    g0 = g0_flops / (stage_ms["expert_up"] * 1e-3) / 1e12
    g1 = g1_flops / (stage_ms["expert_down"] * 1e-3) / 1e12
    by = stage_bytes(cfg, m.comb == "separate16")
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian inputs and random-init weights of the layer's shapes)",
        "config": {"workload": f"{cfg.name}: MoE expert layer T={T} d={d} f={f} E={cfg.E} "
                               f"top-{k}" + (f" + {cfg.n_shared} shared f={cfg.f_shared}"
                                             if cfg.n_shared else ""),
                   "T": T, "d": d, "f": f, "E": cfg.E, "k": k,
                   "path": {"fast": "gather fused into layer 0, separate combine" + (
                                " over compact rows (fp16 + power-of-two factor per 32 columns)"
                                if m.comb == "separate16" else ""),
                            "fast32": "gather fused into layer 0, separate combine",
                            "atomic": "gather fused into layer 0, combine fused into layer 1",
                            "reference": "permuted copy of x, separate combine"}[args.path]},
        "pct_of_bf16_peak": round(100 * tflops / peak, 2),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "event_ms_per_step": round(step_ms, 4),
        "stages_ms": {kk: round(v, 4) for kk, v in stage_ms.items()},
        "stage_rates": {
            "expert_up_TFLOPs": round(g0, 1),
            "expert_down_TFLOPs": round(g1, 1),
            **{f"{st}_GBs": round(by[st] / (stage_ms[st] * 1e-3) / 1e9, 1)
               for st in ("route", "permute", "combine")},
        },
        "roofline": {
            "kernel": gemm_kernel_name(cfg, up=True) + (
                " (layer 0 + SwiGLU; main pass and tail-split fixup, the launches the expert_up "
                "events bracket)" if cfg.dtype == "bf16" else
                " (layer 0 + SwiGLU, one fp32 FMA chain per output; the small fp32 layer is not "
                "sized to fill the chip)"),
            "bound": "mfma" if cfg.dtype == "bf16" else "alu",
            "achieved": round(g0, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(g0 / peak, 4),
            "traffic": measured_traffic(cfg),
        },
    }
    if args.protocol_steps > 0:
        # every step after a 1 GiB write that evicts the last-level cache:
        # median, p10 and p90 of the per-step event times, and the
        # memory-bound stages' HBM rates (fraction of 8 TB/s) at the medians
        per, step = protocol_times(m, args.protocol_steps, 1 << 30)
        med = {st: pct(v, 50) for st, v in per.items()}
        rd = {st: flushed_read_ms(by[st]) for st in ("route", "permute", "combine")}
        out["protocol"] = {
            "what": f"{args.protocol_steps} steps, each after a 1 GiB device write outside the "
                    "events (last-level cache flushed); HIP events on the launch stream",
            "step_ms": {"median": round(pct(step, 50), 4), "p10": round(pct(step, 10), 4),
                        "p90": round(pct(step, 90), 4)},
            "layer_TFLOPs_at_median": round(flops / (pct(step, 50) * 1e-3) / 1e12, 1),
            "stages_ms_median": {st: round(v, 4) for st, v in med.items()},
            "stages_ms_p10": {st: round(pct(v, 10), 4) for st, v in per.items()},
            "stages_ms_p90": {st: round(pct(v, 90), 4) for st, v in per.items()},
            "hbm_stages": {st: {"bytes": by[st],
                                "GBs": round(by[st] / (med[st] * 1e-3) / 1e9, 1),
                                "frac_of_8TBs": round(by[st] / (med[st] * 1e-3) / 1e9 /
                                                      PEAK_HBM_GBS, 3),
                                # a pure streaming read of the same byte count,
                                # also after a flush: what ramp-up and launch
                                # leave of the bandwidth at this size
                                "pure_read_GBs": round(by[st] / (rd[st] * 1e-3) / 1e9, 1),
                                "frac_of_pure_read": round(rd[st] / med[st], 3)}
                           for st in ("route", "permute", "combine")},
            "expert_up_TFLOPs_at_median": round(g0_flops / (med["expert_up"] * 1e-3) / 1e12, 1),
            "expert_down_TFLOPs_at_median": round(g1_flops / (med["expert_down"] * 1e-3) / 1e12,
                                                  1),
        }
    if args.protocol_steps > 0:
        b2b, alone = route_alone(m)
        out["route_alone"] = {
            "what": "moe_route by itself: 20 calls back to back, and 20 single calls each after a "
                    "1 GiB cache flush (median)",
            "back_to_back_us": round(b2b * 1e3, 2),
            "flushed_us": round(alone * 1e3, 2),
            "flushed_GBs": round(by["route"] / (alone * 1e-3) / 1e9, 1),
            "flushed_frac_of_8TBs": round(by["route"] / (alone * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
        }
    if not args.no_peaks:
        out["measured_peaks"] = measured_peaks()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, layer, args.cpu_target_s)
        rt, n_rt = cpu_routing(cfg, layer)
        gpu_rt = stage_ms["route"] + stage_ms["permute"]
        out["cpu_baseline"]["routing"] = {
            "what": "routing and dispatch alone (logits, top-k, weights, counts, offsets, stable "
                    f"permutation) on all {T} tokens: the oracle against the GPU's route + permute "
                    "calls inside the layer",
            "oracle_s": round(rt, 4),
            "oracle_tokens_per_s": round(T / rt, 1),
            "repetitions": n_rt,
            "gpu_route_permute_ms": round(gpu_rt, 4),
            "gpu_tokens_per_s": round(T / (gpu_rt * 1e-3), 1),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
