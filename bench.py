#!/usr/bin/env python3
"""Benchmark of the routed-expert W4A16 group-32 MoE layer on one MI355X.

A step is one whole layer call (moe_layer_forward: router, permutation,
grouped W4A16 FFN and combine; at decode sizes the gate/up kernel routes the
tokens itself) over one batch of seeded synthetic input with every input
already resident in HBM.  The default workload is the 512-expert, top-10,
hidden-2560, intermediate-640 layer at 8 decode tokens.

Measurement
  * The expert weights are cloned into --layers device copies and step s uses
    copy s % layers, so each step streams its active experts from HBM and not
    from the 256 MB last-level cache (a model runs its layers one after the
    other the same way).
  * value: tokens/s of K one-call steps, the fastest of three ways of
    issuing them: eagerly, replayed as HIP graphs of one step (one graph per
    weight copy), and replayed as one graph of `layers` consecutive steps
    (one per weight copy, as a model replays its layers), each bracketed by
    device synchronisation (config.timing names which).
    Before that the same K steps run eagerly as the four separate calls (moe_route_permute,
    moe_w4a16_gate_up, moe_w4a16_down, moe_combine) with HIP events around
    each, for the per-stage breakdown, and the one-call step must reproduce
    their output bit for bit.  The dominant kernel (gate/up, launched alone
    back to back) gives the roofline.
  * cpu_baseline: the CPU oracle (test infrastructure) timed on this host on
    the same workload, best of a few repeats.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16 matrix, AMD published
DEFAULT_WORKLOAD = "decode_e512_k10_h2560_i640_t8"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=480)
    p.add_argument("--warmup", type=int, default=48)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--tokens", type=int, default=None,
                   help="token count T instead of the workload's (the inputs of a smaller T are the "
                        "first rows of the workload's at the same seed), e.g. the 1/2/4/8 decode sweep")
    p.add_argument("--layers", type=int, default=16, help="device copies of the expert weights")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-graph", action="store_true", help="report the eager loop as value")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-repeats", type=int, default=3)
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB a few times (counter calibration)")
    return p.parse_args(argv)


def copy_probe(mib: int) -> int:
    """A plain copy kernel of known size, for scaling HBM byte counters."""
    import torch

    n = mib << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "dispatches": 4}),
          flush=True)
    return 0


# --------------------------------------------------------------------------- #
# algorithmic work (what the layer must move / compute)
# --------------------------------------------------------------------------- #
def expert_bytes(H: int, I: int) -> tuple[int, int]:
    """Bytes of one expert's w13 and w2: int4 codes + fp16 scales + packed zeros."""
    def mat(N, K):
        return N * K // 2 + N * (K // 32) * 2 + (N // 8) * (K // 32) * 4
    return mat(2 * I, H), mat(H, I)


def layer_work(shape, num_active: int) -> dict:
    w13, w2 = expert_bytes(shape.H, shape.I)
    io = shape.T * shape.H * 2 + shape.T * shape.E * 4 + shape.T * shape.H * 2
    return {
        "w13_bytes_per_expert": w13,
        "w2_bytes_per_expert": w2,
        "layer_bytes": num_active * (w13 + w2) + io,
        "gate_up_bytes": num_active * w13 + shape.T * shape.H * 2,
        "down_bytes": num_active * w2,
        "flops": 6 * shape.T * shape.top_k * shape.H * shape.I,
        "gate_up_flops": 4 * shape.T * shape.top_k * shape.H * shape.I,
    }


# --------------------------------------------------------------------------- #
# HBM traffic from rocprofv3 counters (committed summary, valid for one source)
# --------------------------------------------------------------------------- #
DECODE_MAX_T = 8   # token counts at or below this run the GEMV kernels


def kernel_sources(workload: str) -> list:
    """Sources whose text fixes the FFN kernels a workload runs."""
    from w4a16_group_quantized_amd.inputs import WORKLOADS

    csrc = "w4a16_group_quantized_amd/csrc/"
    main = "ffn_decode.hip" if WORKLOADS[workload].T <= DECODE_MAX_T else "ffn_prefill.hip"
    return [csrc + main, csrc + "common.h"]


def source_sha256(rels: list) -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(workload: str, kernel: str):
    """Bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary.

    profiles/counters_<workload>.md holds lines
      traffic <kernel> fetch_kib=F write_kib=W fetch_scale=a write_scale=b source_sha256=S
    where a and b scale each counter to bytes moved by a plain copy of known
    size.  The figure is returned only while the kernel source still hashes
    to S (otherwise the kernel changed since the counters were taken: None).
    """
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        parts = line.split()
        if len(parts) < 2 or parts[0] != "traffic" or parts[1] != kernel:
            continue
        kv = dict(p.split("=", 1) for p in parts[2:])
        if kv.get("source_sha256") != source_sha256(kernel_sources(workload)):
            return None
        fetch = float(kv["fetch_kib"]) * float(kv["fetch_scale"]) * 1024
        write = float(kv["write_kib"]) * float(kv["write_scale"]) * 1024
        return fetch + write
    return None


# --------------------------------------------------------------------------- #
# CPU baseline: the oracle on this host
# --------------------------------------------------------------------------- #
def cpu_baseline(host: dict, shape, repeats: int) -> dict:
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = 1
    sample_T = shape.T
    sub = host
    if shape.T > 64:  # bounded sample of the same workload: its first 64 tokens
        sample_T = 64
        sub = dict(host)
        sub["logits"] = host["logits"][:64]
        sub["x"] = host["x"][:64]
    best = float("inf")
    for _ in range(max(1, repeats)):
        t0 = time.perf_counter()
        oracle.layer(sub, shape.top_k)
        best = min(best, time.perf_counter() - t0)
    _ = np
    return {
        "value": sample_T / best,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"whole layer on the first {sample_T} tokens of the workload, best of {repeats}, "
                  f"fp64 NumPy (unpack single-threaded, BLAS on {threads} threads), "
                  f"{len(os.sched_getaffinity(0))} host cores visible",
        "seconds": best,
    }


# --------------------------------------------------------------------------- #
# GPU measurement
# --------------------------------------------------------------------------- #
def main(argv=None) -> int:
    args = parse_args(argv)
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build runs the MoE layer on a single MI355X "
              "and has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from w4a16_group_quantized_amd import inputs as synth
    from w4a16_group_quantized_amd import ops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    shape = synth.WORKLOADS[args.workload]
    if args.tokens is not None and args.tokens != shape.T:
        shape = dataclasses.replace(shape, T=args.tokens)
        shape.validate()
    # byte counters were taken at the workload's own token count only
    counters_apply = shape.T == synth.WORKLOADS[args.workload].T
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops.load_library()
    log(f"workload {args.workload}: {shape} on {torch.cuda.get_device_name(dev)}")

    host = synth.make_inputs(shape, args.seed)
    logits = torch.from_numpy(host["logits"]).to(dev)
    x = torch.from_numpy(host["x"]).to(dev)
    w0 = ops.weights_to_device(host, dev)
    copies = [w0] + [{k: v.clone() for k, v in w0.items()} for _ in range(args.layers - 1)]
    per_copy = sum(v.numel() * v.element_size() for v in w0.values())
    log(f"{args.layers} weight copies x {per_copy / 2**30:.2f} GiB on device")

    layer = ops.MoELayer(shape.T, shape.E, shape.top_k, shape.H, shape.I, dev)
    stream = torch.cuda.current_stream()

    def step(i: int, ev=None):
        w = copies[i % args.layers]
        if ev is not None:
            ev[0].record(stream)
        ops.moe_route_permute(logits, shape.top_k, layer.perm_ws, layer.ids, layer.weights,
                              layer.perm)
        if ev is not None:
            ev[1].record(stream)
        ops.moe_w4a16_gate_up(x, shape.top_k, layer.perm, w, layer.ffn_ws)
        if ev is not None:
            ev[2].record(stream)
        ops.moe_w4a16_down(shape.T, shape.top_k, layer.perm, w, layer.y_sorted, layer.ffn_ws)
        if ev is not None:
            ev[3].record(stream)
        ops.moe_combine(layer.y_sorted, layer.weights, layer.perm["slot_rows"], layer.out)
        if ev is not None:
            ev[4].record(stream)

    # warm-up (eager), then the eager timed pass with per-call events
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ref_out = layer.out.clone()
    num_active = int(layer.perm["num_active"].item())
    work = layer_work(shape, num_active)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i, evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    eager_ms = t_start.elapsed_time(t_end) / args.steps
    seg = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])  # ms
    seg_ms = seg.mean(axis=0)
    log(f"eager: {eager_ms * 1e3:.1f} us/step; route+permute {seg_ms[0] * 1e3:.1f}, "
        f"gate_up {seg_ms[1] * 1e3:.1f}, down {seg_ms[2] * 1e3:.1f}, combine {seg_ms[3] * 1e3:.1f} us")
    assert torch.equal(layer.out, ref_out), "eager steps disagree"

    # The dominant kernels alone: back-to-back launches on the routing of the
    # batch (left in the layer's buffers), each on the next weight copy.
    def kernel_avg_ms(launch) -> float:
        for i in range(4):
            launch(i)
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        k0.record(stream)
        for i in range(args.steps):
            launch(i)
        k1.record(stream)
        torch.cuda.synchronize()
        return k0.elapsed_time(k1) / args.steps

    gate_up_ms = kernel_avg_ms(lambda i: ops.moe_w4a16_gate_up(
        x, shape.top_k, layer.perm, copies[i % args.layers], layer.ffn_ws))
    down_ms = kernel_avg_ms(lambda i: ops.moe_w4a16_down(
        shape.T, shape.top_k, layer.perm, copies[i % args.layers], layer.y_sorted, layer.ffn_ws))
    log(f"back-to-back: gate_up {gate_up_ms * 1e3:.1f} us, down {down_ms * 1e3:.1f} us")

    # The timed step: the whole layer as one moe_layer_forward call (which, at
    # decode sizes, routes inside the gate/up kernel); it must give the four
    # calls' output bit for bit.
    def layer_step(i: int):
        layer.forward(logits, x, copies[i % args.layers])

    layer.fused_out.zero_()
    layer_step(0)
    torch.cuda.synchronize()
    assert torch.equal(layer.fused_out, ref_out), "moe_layer_forward differs from the four calls"
    t_start.record(stream)
    for i in range(args.steps):
        layer_step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    fused_eager_ms = t_start.elapsed_time(t_end) / args.steps
    log(f"eager moe_layer_forward: {fused_eager_ms * 1e3:.1f} us/step")

    # Per-step spread of the same eager steps (events around each step), and a
    # labelled hot-cache figure: every step on one weight copy, whose active
    # experts then stay in the last-level cache (not a layer of a model).
    def per_step_us(copy_of) -> np.ndarray:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev[i][0].record(stream)
            layer.forward(logits, x, copies[copy_of(i)])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) * 1e3 for a, b in ev])

    spread = per_step_us(lambda i: i % args.layers)
    hot = per_step_us(lambda i: 0)
    step_pct = {f"p{q}": float(np.percentile(spread, q)) for q in (10, 50, 90)}
    log(f"eager steps p10/p50/p90 {step_pct['p10']:.1f} / {step_pct['p50']:.1f} / "
        f"{step_pct['p90']:.1f} us; hot-cache (one weight copy) p50 {np.median(hot):.1f} us")

    # HIP graphs: one captured step per weight copy, replayed round-robin
    graph_ms = None
    graph_multi_ms = None
    if not args.no_graph:
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            for c in range(args.layers):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    layer_step(c)
                graphs.append(g)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        for rep in range(3):  # every replay must reproduce the eager result
            layer.fused_out.zero_()
            graphs[rep % args.layers].replay()
            torch.cuda.synchronize()
            assert torch.equal(layer.fused_out, ref_out), "graph replay differs from eager"
        for i in range(args.warmup):
            graphs[i % args.layers].replay()
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(args.steps):
            graphs[i % args.layers].replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        graph_ms = t_start.elapsed_time(t_end) / args.steps
        assert torch.equal(layer.fused_out, ref_out), "graph replay differs from eager"
        log(f"graph: {graph_ms * 1e3:.1f} us/step")

        # A model step as one graph: `layers` consecutive layer steps (one per
        # weight copy) captured together, as a decoder replays all its layers.
        multi = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(multi, stream=cap):
                for c in range(args.layers):
                    layer_step(c)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        layer.fused_out.zero_()
        multi.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.fused_out, ref_out), "multi-layer graph differs from eager"
        reps = max(1, args.steps // args.layers)
        for _ in range(max(1, args.warmup // args.layers)):
            multi.replay()
        torch.cuda.synchronize()
        t_start.record(stream)
        for _ in range(reps):
            multi.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        graph_multi_ms = t_start.elapsed_time(t_end) / (reps * args.layers)
        log(f"graph of {args.layers} layer steps: {graph_multi_ms * 1e3:.1f} us/step")

    # the fastest of the ways of issuing the same K steps (the per-step
    # HIP-graph replay pays a graph launch per step; the multi-layer graph
    # counts only when K is a whole number of its replays)
    options = {"eager": fused_eager_ms}
    if graph_ms is not None:
        options["hip-graph replay"] = graph_ms
    if graph_multi_ms is not None and args.steps % args.layers == 0:
        options[f"hip-graph replay of {args.layers} layer steps"] = graph_multi_ms
    timing = min(options, key=options.get)
    ms = options[timing]
    tokens_per_s = shape.T / (ms * 1e-3)
    gate_up_s = gate_up_ms * 1e-3
    intensity = work["gate_up_flops"] / work["gate_up_bytes"]
    ridge = MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": work["gate_up_bytes"] / gate_up_s / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": work["gate_up_flops"] / gate_up_s / 1e12,
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = counter_traffic(args.workload, "gate_up") if counters_apply else None
    roof.update({
        "kernel": "gate/up kernel of moe_w4a16_gate_up",
        "avg_launch_us": gate_up_ms * 1e3,
        "algorithmic_bytes_per_launch": work["gate_up_bytes"],
        "algorithmic_flops_per_launch": work["gate_up_flops"],
    })
    result = {
        "metric": "MoE layer tokens/s (decode: HBM GB/s of the gate/up kernel in roofline)",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "w4a16 (int4 weights, fp16 activations, fp32 accumulation)",
        "data": "synthetic (seeded; weights random uint4 codes/zeros, fp16 scales U[0.002,0.02))",
        "config": {
            "workload": args.workload,
            "E": shape.E, "top_k": shape.top_k, "H": shape.H, "I": shape.I, "T": shape.T,
            "group_size": 32, "weight_copies": args.layers, "active_experts": num_active,
            "timing": timing,
        },
        "roofline": roof,
        "layer": {
            "eager_us_per_step": eager_ms * 1e3,
            "eager_layer_forward_us_per_step": fused_eager_ms * 1e3,
            "eager_step_us_percentiles": step_pct,
            "hot_cache_us_per_step_p50": float(np.median(hot)),
            "graph_us_per_step": graph_ms * 1e3 if graph_ms is not None else None,
            "graph_multi_layer_us_per_step": (graph_multi_ms * 1e3 if graph_multi_ms is not None
                                              else None),
            "algorithmic_bytes": work["layer_bytes"],
            "layer_GBps": work["layer_bytes"] / (ms * 1e-3) / 1e9,
            "layer_hbm_frac": work["layer_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "flops": work["flops"],
            "TFLOPs": work["flops"] / (ms * 1e-3) / 1e12,
            "mfma_frac": work["flops"] / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "segments_us": {"route+permute": seg_ms[0] * 1e3, "gate_up": seg_ms[1] * 1e3,
                            "down": seg_ms[2] * 1e3, "combine": seg_ms[3] * 1e3},
            "down_kernel_us": down_ms * 1e3,
            "down_GBps": work["down_bytes"] / (down_ms * 1e-3) / 1e9,
            "down_traffic": counter_traffic(args.workload, "down") if counters_apply else None,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(host, shape, args.cpu_repeats)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
